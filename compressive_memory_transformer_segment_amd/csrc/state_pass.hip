// State pass: the per-segment terms of the memory recurrence, for every segment of a
// window at once (they depend on the segment's own K and V only; for the delta rule also
// on z_{s-1}, a prefix sum of the key sums).
//
//   dz_s = sum_t sigma(k_t)                                   (Eq. 8, z line)
//   U_s  = sigma(K_s)^T V_s, stored transposed as U_s^T [d_value][d_key]   (Eq. 8)
//   G_s  = sigma(K_s)^T diag(1 / (sigma(K_s) z_{s-1} + eps)) sigma(K_s)   (Eq. 9 rearranged)
//
// Eq. 9 is M_s = M_{s-1} + sigma(K)^T V - sigma(K)^T diag(1/den) sigma(K) M_{s-1}
//             = M_{s-1} - G_s M_{s-1} + U_s,
// an exact rearrangement (associativity of the products) that moves the N-long
// contractions out of the sequential chain: the chain only multiplies d x d matrices.
// (Architecture summary of arXiv 2404.07143, section 3.4 "Compressive Memory", Eq. 8-9.)
//
// bf16 path: sigma(K) is formed in fp32 and split into bf16 hi + lo, so the bf16 matrix
// cores give fp32-accurate sums (V is exact in bf16); G uses hi*hi + hi*lo + lo*hi.
// A segment is cut into `chk` chunks, one workgroup each, and every chunk writes its own
// partial sums with plain stores; the chain kernel (the next launch on the stream, so the
// partials are visible to it) adds them in chunk order, which keeps results deterministic
// without any cross-workgroup synchronisation here.
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kThreads = 256;
constexpr int kSub = 64;                  // tokens per sub-tile

enum Mode { MODE_KEYSUM = 0, MODE_LINEAR = 1, MODE_DELTA = 2 };

struct UnitPos {
  int s_local, bh, b, h, n;
  int64_t tok0;  // first token of the segment in the call
};

__device__ __forceinline__ UnitPos unit_pos(const WindowArgs& a, int u) {
  UnitPos p;
  const int BH = a.B * a.H;
  p.s_local = u / BH;
  p.bh = u % BH;
  p.b = p.bh / a.H;
  p.h = p.bh % a.H;
  p.n = a.seg_tokens(p.s_local);
  p.tok0 = static_cast<int64_t>(a.s0 + p.s_local) * a.N;
  return p;
}

// z_{s-1} for unit (s_local, bh): the state's z plus the key sums of the window's earlier
// segments, added segment by segment and chunk by chunk (the chain adds them in the same
// order, so both see the same z).
template <int D>
__device__ void z_before(const WindowArgs& a, const UnitPos& p, float* zs) {
  const int BH = a.B * a.H;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float z = a.zero_state ? 0.f : a.z[static_cast<int64_t>(p.bh) * D + d];
    for (int s = 0; s < p.s_local; ++s) {
      float dz = 0.f;
      for (int c = 0; c < a.chk; ++c) dz += a.ws.dz[((static_cast<int64_t>(s) * BH + p.bh) * a.chk + c) * D + d];
      z += dz;
    }
    zs[d] = z;
  }
}

// Key sums only (the delta rule needs z_{s-1} before its state pass): one workgroup per
// (unit, chunk), 64-token sub-tiles of K loaded three ahead of the one being summed (four
// register sets; the sub-tile loop is unrolled by four, so each set is a fixed register
// range and the compiler waits only for the oldest); each thread sums sigma(K) over its rows
// and 8 features, then the row groups are reduced in group order.
template <int D>
__global__ __launch_bounds__(kThreads) void k_keysum_bf16(const WindowArgs a) {
  constexpr int DQ = D / 8;              // threads per token row (8 features each)
  constexpr int TQ = kThreads / DQ;      // row groups
  constexpr int RPT = kSub / TQ;         // rows per thread per sub-tile
  __shared__ float red[TQ][D];

  const int u = blockIdx.x / a.chk;
  const int c = blockIdx.x % a.chk;
  const UnitPos p = unit_pos(a, u);
  const int tid = threadIdx.x;
  const int dq = tid % DQ, tq = tid / DQ;
  const int64_t seg_base = (static_cast<int64_t>(p.bh) * a.T + p.tok0) * D;
  const int t_begin = c * a.ch;
  const int t_end = min(t_begin + a.ch, p.n);
  // rows past the chunk end read as zeros (the buffer range); they are skipped below
  const auto krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + seg_base, static_cast<uint32_t>(max(t_end, 0)) * D * 2);

  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;
  auto load = [&](int ts, u32x4 (&kd)[RPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      kd[r] = buffer_ld16(krs, (static_cast<uint32_t>(ts + tq * RPT + r) * D + dq * 8) * 2);
  };
  auto add = [&](int ts, const u32x4 (&kd)[RPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      if (ts + tq * RPT + r < t_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zacc[2 * i] += elu_plus_one(bf16lo_to_f32(kd[r][i]));
          zacc[2 * i + 1] += elu_plus_one(bf16hi_to_f32(kd[r][i]));
        }
      }
    }
  };
  // sub-tiles past the chunk end load zeros (their rows are skipped): every load is issued
  const int nsub = t_end > t_begin ? ((t_end - t_begin + 4 * kSub - 1) / (4 * kSub)) * 4 : 0;
  u32x4 k0[RPT], k1[RPT], k2[RPT], k3[RPT];
  if (nsub > 0) {
    load(t_begin, k0);
    load(t_begin + kSub, k1);
    load(t_begin + 2 * kSub, k2);
  }
  for (int i = 0; i < nsub; i += 4) {
    const int ts = t_begin + i * kSub;
    load(ts + 3 * kSub, k3);
    add(ts, k0);
    load(ts + 4 * kSub, k0);
    add(ts + kSub, k1);
    load(ts + 5 * kSub, k1);
    add(ts + 2 * kSub, k2);
    load(ts + 6 * kSub, k2);
    add(ts + 3 * kSub, k3);
  }
  const int64_t slot = static_cast<int64_t>(u) * a.chk + c;
#pragma unroll
  for (int i = 0; i < 8; ++i) red[tq][dq * 8 + i] = zacc[i];
  __syncthreads();
  for (int d = tid; d < D; d += kThreads) {
    float sum = 0.f;
    for (int g = 0; g < TQ; ++g) sum += red[g][d];
    a.ws.dz[slot * D + d] = sum;
  }
}

// Linear rule, bf16 inputs: a warp-specialised pass.  Waves 0-7
// produce (two per SIMD, so that each SIMD has independent exponential chains to
// interleave) and waves 8-11 consume.  Per 64-token stage the producers turn K into sigma(K),
// split into bf16 hi + lo, and stage it with V in LDS, two stages deep; meanwhile the
// consumers accumulate U^T += V^T sigma(K) on the matrix cores from the other stage, so
// the exponentials and the products run side by side.  Producers keep their global loads
// three stages ahead in four register sets; the stage count is rounded up to a multiple
// of four (rows past the chunk end read as zeros and add nothing), so the loop body is
// straight-line code and the compiler's load waits stay exact.  One barrier per stage.
// Every workgroup writes its own partial sums, one slot per (unit, chunk), added in chunk
// order by the chain.
constexpr int kProdWaves = 8;
constexpr int kLinThreads = 64 * (kProdWaves + 4);
template <int D>
__global__ __launch_bounds__(kLinThreads, 1) void k_state_lin_bf16(const WindowArgs a) {
  constexpr int P = D + 32;              // LDS row pitch (elements): conflict-free transpose reads
  constexpr int DQ = D / 8;              // producer threads per token row (8 features each)
  constexpr int TQ = 64 * kProdWaves / DQ;   // producer row groups
  constexpr int RPT = kSub / TQ;         // rows per producer thread per stage
  constexpr int BB = D / 64;             // 32x32 output blocks per consumer wave, per dimension
  __shared__ __align__(16) uint16_t hi_s[2][kSub][P];
  __shared__ __align__(16) uint16_t lo_s[2][kSub][P];
  __shared__ __align__(16) uint16_t v_s[2][kSub][P];
  __shared__ float red[TQ][D];

  const int u = blockIdx.x / a.chk;
  const int c = blockIdx.x % a.chk;
  const UnitPos p = unit_pos(a, u);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int t_begin = c * a.ch;
  const int t_end = min(t_begin + a.ch, p.n);
  const int ns = t_end > t_begin ? ((t_end - t_begin + 4 * kSub - 1) / (4 * kSub)) * 4 : 0;   // stages
  const int64_t slot = static_cast<int64_t>(u) * a.chk + c;
  const int64_t DD = static_cast<int64_t>(D) * D;

  if (wave < kProdWaves) {
    // ---------------------------------------------------------------- producers
    const int dq = tid % DQ, tq = tid / DQ;
    // the segment's K and V rows up to the chunk end; rows past it read as zeros (V = 0
    // there, so the padded rows add nothing to U; the key sums skip them)
    const int64_t seg_base = (static_cast<int64_t>(p.bh) * a.T + p.tok0) * D;
    const auto krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + seg_base, static_cast<uint32_t>(t_end) * D * 2);
    const auto vrs = buffer_rsrc(static_cast<const uint16_t*>(a.v) + seg_base, static_cast<uint32_t>(t_end) * D * 2);
    float zacc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zacc[i] = 0.f;
    auto load = [&](int s, u32x4 (&kd)[RPT], u32x4 (&vd)[RPT]) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const uint32_t off = (static_cast<uint32_t>(t_begin + s * kSub + tq * RPT + r) * D + dq * 8) * 2;
        kd[r] = buffer_ld16(krs, off);
        vd[r] = buffer_ld16(vrs, off);
      }
    };
    // stage s: sigma(K) hi / lo and V into LDS buffer s % 2, key sums of the real rows
    auto convert = [&](int s, const u32x4 (&kd)[RPT], const u32x4 (&vd)[RPT]) __attribute__((always_inline)) {
      const int b = s & 1;
      const int ts = t_begin + s * kSub;
      const bool whole = ts + kSub <= t_end;   // wave-uniform: no padded rows in this stage
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int tl = tq * RPT + r;
        float sk[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sk[2 * i] = elu_plus_one(bf16lo_to_f32(kd[r][i]));
          sk[2 * i + 1] = elu_plus_one(bf16hi_to_f32(kd[r][i]));
        }
        if (whole || ts + tl < t_end) {
#pragma unroll
          for (int i = 0; i < 8; ++i) zacc[i] += sk[i];
        }
        u32x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = pack_bf16x2(sk[2 * i], sk[2 * i + 1]);
          lo[i] = pack_bf16x2(sk[2 * i] - bf16lo_to_f32(hi[i]), sk[2 * i + 1] - bf16hi_to_f32(hi[i]));
        }
        st16(&hi_s[b][tl][dq * 8], hi);
        st16(&lo_s[b][tl][dq * 8], lo);
        st16(&v_s[b][tl][dq * 8], vd[r]);
      }
    };
    // stage s waits in register set s % 4 from its load until its conversion; step i
    // stages i + 1 into the buffer the consumers read in step i - 1
    u32x4 k0[RPT], v0[RPT], k1[RPT], v1[RPT], k2[RPT], v2[RPT], k3[RPT], v3[RPT];
    if (ns > 0) {
      load(0, k0, v0);
      load(1, k1, v1);
      load(2, k2, v2);
      load(3, k3, v3);
      convert(0, k0, v0);
      load(4, k0, v0);
    }
    __syncthreads();   // stage 0 staged
    for (int i = 0; i < ns; i += 4) {
      convert(i + 1, k1, v1);
      load(i + 5, k1, v1);
      __syncthreads();
      convert(i + 2, k2, v2);
      load(i + 6, k2, v2);
      __syncthreads();
      convert(i + 3, k3, v3);
      load(i + 7, k3, v3);
      __syncthreads();
      convert(i + 4, k0, v0);
      load(i + 8, k0, v0);
      __syncthreads();
    }
    // key sums: reduce the per-thread partials over the row groups (in group order)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tq][dq * 8 + i] = zacc[i];
  } else {
    // ---------------------------------------------------------------- consumers
    // consumer wave cw owns the BB x BB blocks (ib0 + bi, jb0 + bj) of U^T
    const int cw = wave - kProdWaves;
    const int ib0 = BB * (cw >> 1), jb0 = BB * (cw & 1);
    f32x16 acc[BB][BB];
#pragma unroll
    for (int bi = 0; bi < BB; ++bi)
#pragma unroll
      for (int bj = 0; bj < BB; ++bj) acc[bi][bj] = zero16();
    __syncthreads();   // stage 0 staged
    // operands of one 16-token k-step: V^T rows (av), sigma(K) hi and lo columns
    struct Ops {
      bf16x8 av[BB], bh[BB], bl[BB];
    };
    auto fetch = [&](int b, int ks, Ops& o) __attribute__((always_inline)) {
#pragma unroll
      for (int bi = 0; bi < BB; ++bi) o.av[bi] = lds_operand_tr(&v_s[b][0][0], P, 16 * ks, 32 * (ib0 + bi), lane);
#pragma unroll
      for (int bj = 0; bj < BB; ++bj) {
        o.bh[bj] = lds_operand_tr(&hi_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
        o.bl[bj] = lds_operand_tr(&lo_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
      }
    };
    auto multiply = [&](const Ops& o) __attribute__((always_inline)) {
#pragma unroll
      for (int bi = 0; bi < BB; ++bi)
#pragma unroll
        for (int bj = 0; bj < BB; ++bj) {
          acc[bi][bj] = mfma32x32x16(o.av[bi], o.bh[bj], acc[bi][bj]);
          acc[bi][bj] = mfma32x32x16(o.av[bi], o.bl[bj], acc[bi][bj]);
        }
    };
    static_assert(kSub == 64, "four k-steps per stage");
    for (int i = 0; i < ns; ++i) {
      // the operands of k-step ks + 2 are read while k-step ks multiplies
      const int b = i & 1;
      Ops o0, o1;
      fetch(b, 0, o0);
      fetch(b, 1, o1);
      __builtin_amdgcn_sched_barrier(0);
      multiply(o0);
      fetch(b, 2, o0);
      __builtin_amdgcn_sched_barrier(0);
      multiply(o1);
      fetch(b, 3, o1);
      __builtin_amdgcn_sched_barrier(0);
      multiply(o0);
      multiply(o1);
      __syncthreads();
    }
    // U^T partial: register r of block (ib, jb) holds row 32 ib + 8 (r / 4) + 4 (lane / 32)
    // + r % 4, column 32 jb + lane % 32
    float* u_dst = a.ws.u + slot * DD;
    const int hl = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int bi = 0; bi < BB; ++bi)
#pragma unroll
      for (int bj = 0; bj < BB; ++bj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * (ib0 + bi) + 8 * (r >> 2) + 4 * hl + (r & 3);
          u_dst[row * D + 32 * (jb0 + bj) + l32] = acc[bi][bj][r];
        }
  }
  __syncthreads();   // the producers' key-sum partials are in red
  for (int d = tid; d < D; d += kLinThreads) {
    float sum = 0.f;
    for (int g = 0; g < TQ; ++g) sum += red[g][d];
    a.ws.dz[slot * D + d] = sum;
  }
}

// Delta rule, bf16 inputs: the warp-specialised layout of k_state_lin_bf16 with the Gram
// term.  Waves 0-3 produce: per 32-token stage they form sigma(K), the row weights
// 1 / (sigma(k_t) . z_{s-1} + eps) and sigma(K) scaled by them, split both into bf16 hi + lo,
// and stage them with V in LDS, two stages deep (their global loads run three stages
// ahead in registers).  Waves 4-7 consume: each owns a 2 x 2 group of 32 x 32 blocks of U^T
// (hi and lo MFMAs) and of G (hi*hi + hi*lo + lo*hi).  One barrier per stage; the stage
// count is rounded up to a multiple of four as in the linear kernel.  The key sums are the
// key-sum pass's: this kernel reads them (z_{s-1}) and must not rewrite them, since other
// workgroups read them concurrently.
constexpr int kSubD = 32;                 // tokens per stage
template <int D>
__global__ __launch_bounds__(512, 1) void k_state_delta_bf16(const WindowArgs a) {
  constexpr int P = D + 32;              // LDS row pitch (elements): conflict-free transpose reads
  constexpr int DQ = D / 8;              // producer threads per token row (8 features each)
  constexpr int TQ = 256 / DQ;           // producer row groups
  constexpr int RPT = kSubD / TQ;        // rows per producer thread per stage
  constexpr int BB = D / 64;             // 32x32 blocks per consumer wave, per dimension
  static_assert(RPT >= 1, "a producer thread owns at least one row");
  __shared__ __align__(16) uint16_t hi_s[2][kSubD][P];
  __shared__ __align__(16) uint16_t lo_s[2][kSubD][P];
  __shared__ __align__(16) uint16_t dh_s[2][kSubD][P];
  __shared__ __align__(16) uint16_t dl_s[2][kSubD][P];
  __shared__ __align__(16) uint16_t v_s[2][kSubD][P];
  __shared__ float zprev[D];

  const int u = blockIdx.x / a.chk;
  const int c = blockIdx.x % a.chk;
  const UnitPos p = unit_pos(a, u);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int t_begin = c * a.ch;
  const int t_end = min(t_begin + a.ch, p.n);
  const int ns = t_end > t_begin ? ((t_end - t_begin + 4 * kSubD - 1) / (4 * kSubD)) * 4 : 0;   // stages
  const int64_t slot = static_cast<int64_t>(u) * a.chk + c;
  const int64_t DD = static_cast<int64_t>(D) * D;

  z_before<D>(a, p, zprev);
  __syncthreads();

  if (wave < 4) {
    // ---------------------------------------------------------------- producers
    const int dq = tid % DQ, tq = tid / DQ;
    const int64_t seg_base = (static_cast<int64_t>(p.bh) * a.T + p.tok0) * D;
    const auto krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + seg_base, static_cast<uint32_t>(t_end) * D * 2);
    const auto vrs = buffer_rsrc(static_cast<const uint16_t*>(a.v) + seg_base, static_cast<uint32_t>(t_end) * D * 2);
    float zp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zp[i] = zprev[dq * 8 + i];
    auto load = [&](int s, u32x4 (&kd)[RPT], u32x4 (&vd)[RPT]) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const uint32_t off = (static_cast<uint32_t>(t_begin + s * kSubD + tq * RPT + r) * D + dq * 8) * 2;
        kd[r] = buffer_ld16(krs, off);
        vd[r] = buffer_ld16(vrs, off);
      }
    };
    auto split = [&](const float (&x)[8], u32x4& hi, u32x4& lo) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        lo[i] = pack_bf16x2(x[2 * i] - bf16lo_to_f32(hi[i]), x[2 * i + 1] - bf16hi_to_f32(hi[i]));
      }
    };
    auto convert = [&](int s, const u32x4 (&kd)[RPT], const u32x4 (&vd)[RPT]) __attribute__((always_inline)) {
      const int b = s & 1;
      const int ts = t_begin + s * kSubD;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int tl = tq * RPT + r;
        const bool real = ts + tl < t_end;
        float sk[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sk[2 * i] = elu_plus_one(bf16lo_to_f32(kd[r][i]));
          sk[2 * i + 1] = elu_plus_one(bf16hi_to_f32(kd[r][i]));
        }
        // den_t = sigma(k_t) . z_{s-1} + eps; the row is spread over DQ consecutive lanes
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) part += sk[i] * zp[i];
#pragma unroll
        for (int off = DQ / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        const float dsc = real ? 1.f / (part + a.eps) : 0.f;
        float dk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) dk[i] = sk[i] * dsc;
        u32x4 hi, lo, dh, dl;
        split(sk, hi, lo);
        split(dk, dh, dl);
        st16(&hi_s[b][tl][dq * 8], hi);
        st16(&lo_s[b][tl][dq * 8], lo);
        st16(&dh_s[b][tl][dq * 8], dh);
        st16(&dl_s[b][tl][dq * 8], dl);
        st16(&v_s[b][tl][dq * 8], vd[r]);
      }
    };
    u32x4 k0[RPT], v0[RPT], k1[RPT], v1[RPT], k2[RPT], v2[RPT], k3[RPT], v3[RPT];
    if (ns > 0) {
      load(0, k0, v0);
      load(1, k1, v1);
      load(2, k2, v2);
      load(3, k3, v3);
      convert(0, k0, v0);
      load(4, k0, v0);
    }
    __syncthreads();   // stage 0 staged
    for (int i = 0; i < ns; i += 4) {
      convert(i + 1, k1, v1);
      load(i + 5, k1, v1);
      __syncthreads();
      convert(i + 2, k2, v2);
      load(i + 6, k2, v2);
      __syncthreads();
      convert(i + 3, k3, v3);
      load(i + 7, k3, v3);
      __syncthreads();
      convert(i + 4, k0, v0);
      load(i + 8, k0, v0);
      __syncthreads();
    }
  } else {
    // ---------------------------------------------------------------- consumers
    const int cw = wave - 4;
    const int ib0 = BB * (cw >> 1), jb0 = BB * (cw & 1);
    f32x16 acc_u[BB][BB], acc_g[BB][BB];
#pragma unroll
    for (int bi = 0; bi < BB; ++bi)
#pragma unroll
      for (int bj = 0; bj < BB; ++bj) {
        acc_u[bi][bj] = zero16();
        acc_g[bi][bj] = zero16();
      }
    __syncthreads();   // stage 0 staged
    for (int i = 0; i < ns; ++i) {
      const int b = i & 1;
#pragma unroll
      for (int ks = 0; ks < kSubD / 16; ++ks) {
        bf16x8 av[BB], ah[BB], al[BB], bh[BB], bl[BB], eh[BB], el[BB];
#pragma unroll
        for (int bi = 0; bi < BB; ++bi) {
          av[bi] = lds_operand_tr(&v_s[b][0][0], P, 16 * ks, 32 * (ib0 + bi), lane);
          ah[bi] = lds_operand_tr(&hi_s[b][0][0], P, 16 * ks, 32 * (ib0 + bi), lane);
          al[bi] = lds_operand_tr(&lo_s[b][0][0], P, 16 * ks, 32 * (ib0 + bi), lane);
        }
#pragma unroll
        for (int bj = 0; bj < BB; ++bj) {
          bh[bj] = lds_operand_tr(&hi_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
          bl[bj] = lds_operand_tr(&lo_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
          eh[bj] = lds_operand_tr(&dh_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
          el[bj] = lds_operand_tr(&dl_s[b][0][0], P, 16 * ks, 32 * (jb0 + bj), lane);
        }
#pragma unroll
        for (int bi = 0; bi < BB; ++bi)
#pragma unroll
          for (int bj = 0; bj < BB; ++bj) {
            // U^T block: rows = value features, columns = key features
            acc_u[bi][bj] = mfma32x32x16(av[bi], bh[bj], acc_u[bi][bj]);
            acc_u[bi][bj] = mfma32x32x16(av[bi], bl[bj], acc_u[bi][bj]);
            // G block: rows = key features (sigma(K)), columns = key features (scaled)
            acc_g[bi][bj] = mfma32x32x16(ah[bi], eh[bj], acc_g[bi][bj]);
            acc_g[bi][bj] = mfma32x32x16(ah[bi], el[bj], acc_g[bi][bj]);
            acc_g[bi][bj] = mfma32x32x16(al[bi], eh[bj], acc_g[bi][bj]);
          }
      }
      __syncthreads();
    }
    float* u_dst = a.ws.u + slot * DD;
    float* g_dst = a.ws.g + slot * DD;
    const int hl = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int bi = 0; bi < BB; ++bi)
#pragma unroll
      for (int bj = 0; bj < BB; ++bj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * (ib0 + bi) + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int col = 32 * (jb0 + bj) + l32;
          u_dst[row * D + col] = acc_u[bi][bj][r];
          g_dst[row * D + col] = acc_g[bi][bj][r];
        }
  }
}

// ------------------------------------------------------------------ float32 I/O path
// One workgroup per unit (no chunking).  Thread (bi, bj) owns a TB x TB block of U (and
// G); tokens are staged in LDS 32 at a time.
template <int D, bool DELTA>
__global__ __launch_bounds__(kThreads) void k_state_f32(const WindowArgs a) {
  constexpr int TB = D / 16;
  constexpr int TT = 32;
  __shared__ float sk[TT][D];
  __shared__ float vv[TT][D];
  __shared__ float dsc[TT];
  __shared__ float zprev[D];

  const int u = blockIdx.x;
  const UnitPos p = unit_pos(a, u);
  const int tid = threadIdx.x;
  const int bi = tid / 16, bj = tid % 16;
  if (DELTA) z_before<D>(a, p, zprev);

  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);
  const int64_t base = (static_cast<int64_t>(p.bh) * a.T + p.tok0) * D;

  float accu[TB][TB], accg[TB][TB];
  for (int i = 0; i < TB; ++i)
    for (int j = 0; j < TB; ++j) accu[i][j] = accg[i][j] = 0.f;
  float zsum = 0.f;

  for (int t0 = 0; t0 < p.n; t0 += TT) {
    __syncthreads();
    for (int e = tid; e < TT * D; e += kThreads) {
      const int t = e / D, d = e % D;
      const bool ok = t0 + t < p.n;
      sk[t][d] = ok ? elu_plus_one(kg[base + static_cast<int64_t>(t0 + t) * D + d]) : 0.f;
      vv[t][d] = ok ? vg[base + static_cast<int64_t>(t0 + t) * D + d] : 0.f;
    }
    __syncthreads();
    if (DELTA && tid < TT) {
      float den = 0.f;
      for (int d = 0; d < D; ++d) den += sk[tid][d] * zprev[d];
      dsc[tid] = 1.f / (den + a.eps);
    }
    if (tid < D)
      for (int t = 0; t < TT; ++t) zsum += sk[t][tid];
    __syncthreads();
    for (int t = 0; t < TT; ++t) {
      float ks[TB], vs[TB], ds[TB];
      for (int i = 0; i < TB; ++i) {
        ks[i] = sk[t][bi * TB + i];
        vs[i] = vv[t][bj * TB + i];
        if (DELTA) ds[i] = sk[t][bj * TB + i] * dsc[t];
      }
      for (int i = 0; i < TB; ++i)
        for (int j = 0; j < TB; ++j) {
          accu[i][j] += ks[i] * vs[j];
          if (DELTA) accg[i][j] += ks[i] * ds[j];
        }
    }
  }
  const int64_t DD = static_cast<int64_t>(D) * D;
  for (int i = 0; i < TB; ++i)
    for (int j = 0; j < TB; ++j) {
      // U^T [value feature][key feature]; G [key feature][key feature]
      const int64_t e = static_cast<int64_t>(bi * TB + i) * D + bj * TB + j;
      const int64_t et = static_cast<int64_t>(bj * TB + j) * D + bi * TB + i;
      a.ws.u[u * DD + et] = accu[i][j];
      if (DELTA) a.ws.g[u * DD + e] = accg[i][j];
    }
  if (!DELTA && tid < D) a.ws.dz[static_cast<int64_t>(u) * D + tid] = zsum;   // chk == 1
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_keysum_f32(const WindowArgs a) {
  const int u = blockIdx.x;
  const UnitPos p = unit_pos(a, u);
  const float* kg = static_cast<const float*>(a.k);
  const int64_t base = (static_cast<int64_t>(p.bh) * a.T + p.tok0) * D;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float s = 0.f;
    for (int t = 0; t < p.n; ++t) s += elu_plus_one(kg[base + static_cast<int64_t>(t) * D + d]);
    a.ws.dz[static_cast<int64_t>(u) * D + d] = s;
  }
}

template <int D>
hipError_t launch_state_d(const WindowArgs& a, hipStream_t st, int mode) {
  if (a.bf16) {
    const dim3 grid(a.units() * a.chk);
    if (mode == MODE_KEYSUM) hipLaunchKernelGGL((k_keysum_bf16<D>), grid, dim3(kThreads), 0, st, a);
    else if (mode == MODE_LINEAR) hipLaunchKernelGGL((k_state_lin_bf16<D>), grid, dim3(kLinThreads), 0, st, a);
    else hipLaunchKernelGGL((k_state_delta_bf16<D>), grid, dim3(512), 0, st, a);
  } else {
    const dim3 grid(a.units());
    if (mode == MODE_KEYSUM) hipLaunchKernelGGL((k_keysum_f32<D>), grid, dim3(kThreads), 0, st, a);
    else if (mode == MODE_LINEAR) hipLaunchKernelGGL((k_state_f32<D, false>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_state_f32<D, true>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_key_sums(const WindowArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_state_d<128>(a, st, MODE_KEYSUM) : launch_state_d<64>(a, st, MODE_KEYSUM);
}

hipError_t launch_state_pass(const WindowArgs& a, hipStream_t st) {
  const int mode = a.delta ? MODE_DELTA : MODE_LINEAR;
  return a.D == 128 ? launch_state_d<128>(a, st, mode) : launch_state_d<64>(a, st, mode);
}

}  // namespace infini
