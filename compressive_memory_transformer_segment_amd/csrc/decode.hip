// Incremental decoding of the Infini-attention layer: one new token per (batch element,
// head) per launch, inside the current segment (the architecture summary of
// arXiv 2404.07143, section 1 on streaming inference and section 3.4's segment-wise
// recurrence, Eq. 4).  For the token at position p of segment s:
//
//   A_dot = softmax(scale * q [K_s[0..p]]^T) V_s[0..p]            (Eq. 6, its row p)
//   A_mem = sigma(q) M_{s-1} / (sigma(q) z_{s-1} + eps)            (Eq. 7)
//   out   = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot     (Eq. 10)
//
// and the token's key and value are appended to the segment's cache.  The memory is
// written (Eq. 8 / 9) by the state-pass and chain kernels over the cache when the segment
// closes; this kernel only reads M_{s-1}, z_{s-1}.
//
// The work is a read of the segment's cached keys and values (p rows of d each) and of
// M_{s-1}: bound by HBM bandwidth.  One workgroup (4 waves) per (batch, head): d/8 lanes
// share a key (8 values per lane, one 16-byte load for bf16), so one wave-wide load covers
// 64/(d/8) keys and is fully coalesced; every lane group keeps its own online-softmax
// state (exp2 domain, scale folded into q) over a strided subset of the keys, and the
// partial states are merged through LDS.  The key loop is double-buffered: the raw loads of
// the next batch of rounds (8 keys per lane group for bf16) are in flight while a batch is
// consumed, and the first batch is issued before the retrieval.  The retrieval reads, with
// bf16 inputs, the bf16 M_{s-1}^T that the forward pass's retrieval uses (the chain keeps it
// next to the fp32 state; one row of 2d bytes per value feature, split over 256 / d
// threads), and with f32 inputs the fp32 M_{s-1} row by row with 16-byte loads.
// With few (batch, head) pairs one workgroup per pair leaves most compute units idle and
// each workgroup streams up to N cached rows alone; the keys are then split into chunks of
// whole key batches over several workgroups per pair (SPLIT).  Each writes its partial
// softmax state with device-coherent stores and counts itself with one atomic; the one that
// counts last merges the chunks in chunk order (the same arithmetic whichever workgroup it
// is) with the retrieval that chunk 0 wrote, and stores the gated output.  Nothing waits.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kDecThreads = 256;

// 8 consecutive elements as float, from bf16 (one 16-byte load) or f32 (two).
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, float (&x)[8]) {
  if constexpr (BF16) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo_to_f32(w[i]);
      x[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  } else {
    const u32x4 w0 = ld16(p), w1 = ld16(static_cast<const float*>(p) + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(w0[i]);
      x[4 + i] = __uint_as_float(w1[i]);
    }
  }
}

// 8 consecutive elements as loaded (bf16: one 16-byte load; f32: two), converted later.
template <bool BF16>
struct Raw8 {
  u32x4 w[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void* p) {
  Raw8<BF16> r;
  r.w[0] = ld16(p);
  if constexpr (!BF16) r.w[1] = ld16(static_cast<const float*>(p) + 4);
  return r;
}
template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      x[2 * i] = bf16lo_to_f32(r.w[0][i]);
      x[2 * i + 1] = bf16hi_to_f32(r.w[0][i]);
    } else {
      x[i] = __uint_as_float(r.w[0][i]);
      x[4 + i] = __uint_as_float(r.w[1][i]);
    }
  }
}

// x + x of another lane in the same 16-lane row (DPP: no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of G = 8 or 16 lanes, left in every lane of the group: swap
// neighbours (quad_perm 1,0,3,2), pairs (quad_perm 2,3,0,1), quads within 8 lanes
// (row_half_mirror) and, for 16, the 8-lane halves of the row (row_mirror).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  x = dpp_add<0x141>(x);
  if constexpr (G == 16) x = dpp_add<0x140>(x);
  return x;
}

template <int D, bool BF16, bool SPLIT>
__global__ __launch_bounds__(kDecThreads) void k_decode(const DecodeArgs a) {
  using T = std::conditional_t<BF16, uint16_t, float>;
  constexpr int LPK = D / 8;           // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wave per round
  constexpr int NG = 4 * KPW;          // lane groups (keys per round) in the workgroup
  constexpr int RS = kDecThreads * 4 / D;   // row slices of the retrieval (4 columns per thread)
  __shared__ float part_m[NG], part_l[NG];
  __shared__ __align__(16) float part_acc[NG][D];
  __shared__ __align__(16) float sq[D];        // sigma(q)
  __shared__ __align__(16) float red[RS][D];   // retrieval partial sums
  __shared__ float zden[4];
  __shared__ int s_count;

  const int bh = SPLIT ? static_cast<int>(blockIdx.x) / a.nsplit : static_cast<int>(blockIdx.x);
  const int cs = SPLIT ? static_cast<int>(blockIdx.x) - bh * a.nsplit : 0;   // key chunk
  const bool lead = cs == 0;   // appends the token and computes the retrieval
  const int h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * KPW + lane / LPK;   // lane group: keys grp, grp + NG, ...
  const int e = lane % LPK;                  // values 8e .. 8e + 7 of each key
  const T* qg = static_cast<const T*>(a.q) + static_cast<int64_t>(bh) * D;
  const T* kg = static_cast<const T*>(a.k) + static_cast<int64_t>(bh) * D;
  const T* vg = static_cast<const T*>(a.v) + static_cast<int64_t>(bh) * D;
  T* kc = static_cast<T*>(a.kc) + static_cast<int64_t>(bh) * a.N * D;
  T* vc = static_cast<T*>(a.vc) + static_cast<int64_t>(bh) * a.N * D;

  // key loop batches: R rounds of NG keys; key t of the batch rounds is read from the cache
  // for t < p, from the inputs for t == p (this token) and, past the end, from any valid
  // row (the result is not used), so every load is unconditional
  constexpr int R = BF16 ? 8 : 4;
  constexpr int BATCH = NG * R;
  const int nk = a.p + 1;
  const int k_lo = SPLIT ? cs * a.chunk : 0;           // this workgroup's keys [k_lo, k_hi)
  const int k_hi = SPLIT ? min(k_lo + a.chunk, nk) : nk;
  auto load_batch = [&](int r0, Raw8<BF16> (&kb)[R], Raw8<BF16> (&vb)[R]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = r0 + u * NG + grp;
      const T* kr = t < a.p ? kc + static_cast<int64_t>(t) * D : kg;
      const T* vr = t < a.p ? vc + static_cast<int64_t>(t) * D : vg;
      kb[u] = load_raw8<BF16>(kr + 8 * e);
      vb[u] = load_raw8<BF16>(vr + 8 * e);
    }
  };
  Raw8<BF16> kA[R], vA[R], kB[R], vB[R];
  load_batch(k_lo, kA, vA);

  // append the token to the cache (read back by later launches only) and form sigma(q)
  if (tid < D && lead) {
    kc[static_cast<int64_t>(a.p) * D + tid] = kg[tid];
    vc[static_cast<int64_t>(a.p) * D + tid] = vg[tid];
    float qf;
    if constexpr (BF16) qf = bf16_to_f32(qg[tid]);
    else qf = qg[tid];
    sq[tid] = elu_plus_one(qf);
  }

  // ---- retrieval partial sums
  //  f32: thread (slice, column quad) over D / RS rows of M_{s-1}
  //  bf16: thread (slice, value feature dv) over D / NS entries of row dv of M_{s-1}^T
  constexpr int NS = kDecThreads / D;   // bf16: slices
  const int cq = tid % (D / 4), slice = tid / (D / 4);
  constexpr int RPS = D / RS;   // rows per slice
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float numt = 0.f;
  __syncthreads();   // sq
  if (!lead) {
    // (other chunks: no retrieval)
  } else if (!a.zero_state) {
    if constexpr (BF16) {
      const int dv = tid % D, sl = tid / D;
      const uint16_t* row = static_cast<const uint16_t*>(a.mt) + (static_cast<int64_t>(bh) * D + dv) * D + sl * (D / NS);
      u32x4 w[D / NS / 8];
#pragma unroll
      for (int j = 0; j < D / NS / 8; ++j) w[j] = ld16(row + 8 * j);
#pragma unroll
      for (int j = 0; j < D / NS / 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = sl * (D / NS) + 8 * j + 2 * e;
          numt = fmaf(sq[i], bf16lo_to_f32(w[j][e]), numt);
          numt = fmaf(sq[i + 1], bf16hi_to_f32(w[j][e]), numt);
        }
    } else {
      const float* Mb = a.M + static_cast<int64_t>(bh) * D * D + 4 * cq;
#pragma unroll 8
      for (int r = 0; r < RPS; ++r) {
        const int i = slice * RPS + r;
        const u32x4 w = ld16(Mb + static_cast<int64_t>(i) * D);
        const float s = sq[i];
#pragma unroll
        for (int c = 0; c < 4; ++c) num[c] = fmaf(s, __uint_as_float(w[c]), num[c]);
      }
    }
    if (wave == 0) {   // sigma(q) . z_{s-1}
      float zs = 0.f;
      for (int i = lane; i < D; i += 64) zs = fmaf(sq[i], a.z[static_cast<int64_t>(bh) * D + i], zs);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) zs += __shfl_xor(zs, off);
      if (lane == 0) zden[0] = zs;
    }
  } else if (tid == 0) {
    zden[0] = 0.f;
  }
  // (a chunk other than 0 stores zeros here, unused)
  if constexpr (BF16) {
    red[tid / D][tid % D] = numt;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) red[slice][4 * cq + c] = num[c];
  }

  // ---- local attention over keys 0 .. p (key p is this token, from the inputs)
  float qv[8];
  load8<BF16>(qg + 8 * e, qv);
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] *= a.scale_log2;
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  auto consume = [&](int r0, const Raw8<BF16> (&kb)[R], const Raw8<BF16> (&vb)[R]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = r0 + u * NG + grp;
      float kk[8];
      unpack8<BF16>(kb[u], kk);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], kk[i], s);
      s = group_sum<LPK>(s);
      if (t < k_hi) {   // uniform across the lane group
        float vv[8];
        unpack8<BF16>(vb[u], vv);
        const float m_new = fmaxf(m, s);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // m = -inf on the first key: 0
        const float pw = __builtin_amdgcn_exp2f(s - m_new);
        l = fmaf(l, alpha, pw);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(acc[i], alpha, pw * vv[i]);
        m = m_new;
      }
    }
  };
  for (int r0 = k_lo; r0 < k_hi; r0 += 2 * BATCH) {
    load_batch(r0 + BATCH, kB, vB);
    consume(r0, kA, vA);
    load_batch(r0 + 2 * BATCH, kA, vA);
    consume(r0 + BATCH, kB, vB);
  }
  if (e == 0) {
    part_m[grp] = m;
    part_l[grp] = l;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part_acc[grp][8 * e + i] = acc[i];
  __syncthreads();

  // ---- merge the lane groups, gate, store
  if constexpr (!SPLIT) {
  if (tid < D) {
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g) mx = fmaxf(mx, part_m[g]);   // finite: group 0 holds key 0
    float nd = 0.f, dd = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float w = __builtin_amdgcn_exp2f(part_m[g] - mx);   // empty group: exp2(-inf) = 0
      nd = fmaf(w, part_acc[g][tid], nd);
      dd = fmaf(w, part_l[g], dd);
    }
    const float a_dot = nd / dd;
    float nm = 0.f;
#pragma unroll
    for (int sl = 0; sl < (BF16 ? NS : RS); ++sl) nm += red[sl][tid];
    const float a_mem = nm / (zden[0] + a.eps);
    const float o = a.gate_g[h] * a_mem + a.gate_omg[h] * a_dot;
    T* og = static_cast<T*>(a.out) + static_cast<int64_t>(bh) * D;
    if constexpr (BF16) og[tid] = f32_to_bf16(o);
    else og[tid] = o;
  }
  } else {
    // this chunk's partial state into slot cs of the pair (and the retrieval, chunk 0)
    constexpr uint32_t SW = D + 2;   // floats per slot: accumulators, maximum, row sum
    const auto rs = buffer_rsrc(a.sp_part + static_cast<int64_t>(bh) * kDecSlots * SW, kDecSlots * SW * 4u);
    if (tid < D) {
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < NG; ++g) mx = fmaxf(mx, part_m[g]);   // finite: group 0 holds key k_lo
      float nd = 0.f, dd = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float w = __builtin_amdgcn_exp2f(part_m[g] - mx);
        nd = fmaf(w, part_acc[g][tid], nd);
        dd = fmaf(w, part_l[g], dd);
      }
      buffer_st4_dev(rs, (cs * SW + tid) * 4u, nd);
      if (tid == 0) {
        buffer_st4_dev(rs, (cs * SW + D) * 4u, mx);
        buffer_st4_dev(rs, (cs * SW + D + 1) * 4u, dd);
      }
      if (lead) {
        float nm = 0.f;
#pragma unroll
        for (int sl = 0; sl < (BF16 ? NS : RS); ++sl) nm += red[sl][tid];
        buffer_st4_dev(rs, ((kDecSlots - 1) * SW + tid) * 4u, nm);
        if (tid == 0) buffer_st4_dev(rs, ((kDecSlots - 1) * SW + D) * 4u, zden[0]);
      }
    }
    wait_vm_lgkm0<0>();   // this thread's stores have completed
    __syncthreads();      // ... every thread's
    if (tid == 0) s_count = __hip_atomic_fetch_add(a.sp_cnt + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_count != a.nsplit - 1) return;   // another chunk's workgroup merges
    if (tid < D) {
      float mx = -INFINITY;
      for (int c = 0; c < a.nsplit; ++c) mx = fmaxf(mx, buffer_ld4_dev(rs, (c * SW + D) * 4u));
      float nd = 0.f, dd = 0.f;
      for (int c = 0; c < a.nsplit; ++c) {
        const float w = __builtin_amdgcn_exp2f(buffer_ld4_dev(rs, (c * SW + D) * 4u) - mx);
        nd = fmaf(w, buffer_ld4_dev(rs, (c * SW + tid) * 4u), nd);
        dd = fmaf(w, buffer_ld4_dev(rs, (c * SW + D + 1) * 4u), dd);
      }
      const float a_dot = nd / dd;
      const float nm = buffer_ld4_dev(rs, ((kDecSlots - 1) * SW + tid) * 4u);
      const float zd = buffer_ld4_dev(rs, ((kDecSlots - 1) * SW + D) * 4u);
      const float a_mem = nm / (zd + a.eps);
      const float o = a.gate_g[h] * a_mem + a.gate_omg[h] * a_dot;
      T* og = static_cast<T*>(a.out) + static_cast<int64_t>(bh) * D;
      if constexpr (BF16) og[tid] = f32_to_bf16(o);
      else og[tid] = o;
    }
    if (tid == 0) __hip_atomic_store(a.sp_cnt + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const bool split = a.nsplit > 1;
  if (split && (!a.sp_part || !a.sp_cnt || a.nsplit > kDecSplitMax || a.chunk % 128 != 0 ||
                int64_t(a.chunk) * (a.nsplit - 1) >= a.p + 1))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * (split ? a.nsplit : 1))), block(kDecThreads);
  auto go = [&](auto d, auto bf) {
    constexpr int D = decltype(d)::value;
    constexpr bool BF = decltype(bf)::value;
    if (split) hipLaunchKernelGGL((k_decode<D, BF, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_decode<D, BF, false>), grid, block, 0, st, a);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  if (a.D == 128) {
    if (a.bf16) go(I128{}, std::true_type{});
    else go(I128{}, std::false_type{});
  } else if (a.D == 64) {
    if (a.bf16) go(I64{}, std::true_type{});
    else go(I64{}, std::false_type{});
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace infini
