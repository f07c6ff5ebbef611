// Fused per-segment output of the Infini-attention layer (architecture summary of
// arXiv 2404.07143, section 3.4):
//
//   A_dot = softmax(scale * Q K^T, causal inside the segment) V                  (Eq. 6)
//   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)                          (Eq. 7)
//   out   = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot                   (Eq. 10)
//
// One workgroup = 4 waves = 128 queries of one (batch, head, segment); every wave owns 32
// queries.  The kernel works in the transposed frame: S^T = K Q^T and O^T = V^T P^T, so
// that a lane holds one query (lane % 32) in every MFMA result.  Softmax statistics are
// then per-lane scalars (plus one exchange with lane ^ 32), the S^T result registers are
// directly the B operand of O^T += V^T P^T, and the retrieval sigma(Q) reuses the Q
// registers (Q is the B operand of S^T) as the B operand of A_mem^T = M^T sigma(Q)^T.
//
// K and V tiles (64 keys x d) go from HBM straight into LDS with buffer -> LDS copies,
// double buffered: the copy of tile j + 1 (in the last iteration: M^T_{s-1} and z_{s-1})
// is in flight while tile j is consumed, and no registers hold data in transit.  Rows past
// the segment end arrive as zeros (buffer range check), so ragged tails need no branches.
// The V^T operand of O^T += V^T P^T is read with LDS transpose reads, in the key order the
// S^T result registers hold.  The online softmax is in the exp2 domain with the scale
// folded in, and rescales the accumulator lazily: only when a row maximum grows by more
// than 2^8 (exact: the final division uses the same stale maximum).  The gated result is
// staged through LDS and written once with coalesced 16-byte stores.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;   // queries per workgroup (4 waves x 32)
constexpr int kBN = 64;    // keys per tile
constexpr float kTau = 8.f;

template <int N_>
using IC = std::integral_constant<int, N_>;

// Workgroup -> (unit, query tile): query tiles longest first across all units, so the
// many short diagonal-heavy tiles fill the tail of the launch.
template <int BM>
__device__ __forceinline__ void tile_of_block(int units, int nq, int& u, int& qt) {
  const int b = static_cast<int>(blockIdx.x);
  qt = nq - 1 - b / units;
  u = b % units;
}

template <int D, bool PARTS>
__global__ __launch_bounds__(kThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(const WindowArgs a) {
  constexpr int KS = D / 16;                  // k-steps over the head dimension
  constexpr int DB = D / 32;                  // 32-row blocks of the head dimension
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = kBN * D;               // elements of one K or V tile
  constexpr int BUF = 2 * TILE;               // one buffer: [K tile | V tile]
  constexpr int NV = D / 32;                  // 1 KB copies per wave for a V tile
  static_assert(kBM * D <= BUF && D * D <= BUF, "Q, M^T and the output fit in one buffer");

  // LDS layouts (bf16, 16-byte chunks; chunk c of a row holds columns 8c .. 8c + 7):
  //  "row groups" for K, Q and M^T: chunk c of row r sits in slot
  //      (r / 16) * 16 CPR + 16 c + r % 16,
  //  so the 16 rows an MFMA operand read touches at one chunk are 16 consecutive slots
  //  (one 256-byte bank line), and every k-step / row block is an immediate offset;
  //  "quads" for V: chunk c of row r sits in slot (r / 4) * 4 CPR + 4 c + r % 4, so the
  //  4 rows x 64 bytes a transpose read takes per half-wave are 16 consecutive slots.
  // Each layout is filled by 1 KB buffer -> LDS copies (64 lanes x 16 bytes, lane i to
  // slot 64 k + i of copy k); everything that differs between a wave's copies is in the
  // scalar resource base and the LDS base, so one offset register per layout suffices.
  // The output is staged row-major with chunk c of row r at physical chunk c ^ swz(r).
  __shared__ __align__(16) uint16_t buf0[BUF];
  __shared__ __align__(16) uint16_t buf1[BUF];
  __shared__ __align__(16) float zsh[256];

  const int units = a.units();
  const int nq = (a.N + kBM - 1) / kBM;
  int u, qt;
  tile_of_block<kBM>(units, nq, u, qt);
  const int BH = a.B * a.H;
  const int s_local = u / BH, bh = u % BH, h = bh % a.H;
  const int n = a.seg_tokens(s_local);
  const int q0 = qt * kBM;
  if (q0 >= n) return;
  const int64_t tok0 = static_cast<int64_t>(a.s0 + s_local) * a.N;
  const int64_t row0 = static_cast<int64_t>(bh) * a.T + tok0;   // token row of the segment start

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + l32;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + row0 * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + row0 * D;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + row0 * D;

  // source byte offsets of this lane's 16 bytes within a copy:
  //   row groups, copy (g, j): rows 16 g + lane % 16, chunk 4 j + lane / 16
  //   quads, copy k: rows 4 (CPR k / 16 + lane / (4 CPR)) + lane % 4, chunk (lane / 4) % CPR
  const uint32_t lp_g = (lane & 15) * (2 * D) + 16 * (lane >> 4);
  const uint32_t lp_v = (((lane >> 2) / CPR) * 4 + (lane & 3)) * (2 * D) + 16 * ((lane >> 2) % CPR);
  // one copy: the resource starts `shift` bytes into the source (bytes past `bytes` of the
  // source read as zeros), the 1 KB lands at lds
  auto copy1k = [&](const void* src, uint32_t bytes, uint32_t shift, void* lds, uint32_t voff)
      __attribute__((always_inline)) {
    const int left = __builtin_amdgcn_readfirstlane(max(static_cast<int>(bytes) - static_cast<int>(shift), 0));
    buffer_to_lds16(buffer_rsrc(static_cast<const char*>(src) + shift, static_cast<uint32_t>(left)), lds, voff);
  };
  // row-group copies of this wave's GW groups (of 16 rows) of a tile
  auto copy_groups = [&](auto gwc, const void* src, uint32_t bytes, uint16_t* dst) __attribute__((always_inline)) {
    constexpr int GW = decltype(gwc)::value;
#pragma unroll
    for (int gg = 0; gg < GW; ++gg)
#pragma unroll
      for (int j = 0; j < CPR / 4; ++j) {
        const int g = wave * GW + gg;
        copy1k(src, bytes, g * 32 * D + 64 * j, reinterpret_cast<char*>(dst) + (g * (CPR / 4) + j) * 1024, lp_g);
      }
  };
  auto bufp = [&](auto bc) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(bc)::value == 0) return buf0;
    else return buf1;
  };
  const int nkv = (min(q0 + kBM, n) + kBN - 1) / kBN;
  // K and V of tile j; rows at or past the segment end arrive as zeros
  auto load_tile = [&](int j, uint16_t* dst) __attribute__((always_inline)) {
    const int kv0 = j * kBN;
    const uint32_t bytes = static_cast<uint32_t>(n - kv0) * D * 2;
    copy_groups(IC<1>{}, kg + static_cast<int64_t>(kv0) * D, bytes, dst);
    const uint16_t* vsrc = vg + static_cast<int64_t>(kv0) * D;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int k = wave * NV + i;
      copy1k(vsrc, bytes, 1024 * k, reinterpret_cast<char*>(dst + TILE) + 1024 * k, lp_v);
    }
  };
  // M^T_{s-1} ([d_value][d_key]) and z_{s-1} for the epilogue
  auto load_mt = [&](uint16_t* dst) __attribute__((always_inline)) {
    copy_groups(IC<D / 64>{}, static_cast<const uint16_t*>(a.ws.mt) + static_cast<int64_t>(u) * D * D, D * D * 2, dst);
    if (wave == 0)   // lanes past D / 4 read zeros
      copy1k(a.ws.zb + static_cast<int64_t>(u) * D, D * 4, 0, zsh, static_cast<uint32_t>(lane) * 16);
  };
  // element offsets of this lane's operand reads
  //  K / Q / M^T (row groups): row 32 blk + l32, chunk 2 ks + hl
  //    -> g_rd + blk * 256 CPR + ks * 256
  //  V^T (quads, transpose reads): k-slot (hl, i) of k-step j4 is key
  //    16 j4 + 8 (i / 4) + 4 hl + i % 4, the key the S^T register feeding that slot holds;
  //    the lane addresses row 16 j4 + 8 s + 4 hl + (lane % 16) / 4 and columns
  //    32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. +3
  //    -> v_rd + (4 j4 + 2 s) * 32 CPR + db * 128
  const int g_rd = ((l32 >> 4) * 16 * CPR + 16 * hl + (l32 & 15)) * 8;
  const int v_rd = TILE + (hl * 4 * CPR + (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * 4 + ((lane & 15) >> 2)) * 8 +
                   4 * (lane & 1);
  auto swz = [](int row) __attribute__((always_inline)) -> int { return D == 128 ? (row & 15) : ((row >> 1) & 7); };

  // ---- prologue: the Q tile into buffer 1, tile 0 into buffer 0
  u32x4 qreg[KS];
  {
    copy_groups(IC<2>{}, qg + static_cast<int64_t>(q0) * D, static_cast<uint32_t>(n - q0) * D * 2, buf1);
    load_tile(0, buf0);
    __syncthreads();
    // Q as the B operand of S^T: lane holds Q[q][16 ks + 8 hl .. +7]; rows >= n are 0
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = ld16(buf1 + g_rd + wave * 256 * CPR + 256 * ks);
    __syncthreads();   // buffer 1 is free again before tile 1 is copied there
  }

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;   // running row maximum, scaled (log2 domain)
  float l_part = 0.f;        // this lane's half of the row sum
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = zero16();

  // One 64-key tile is processed as two 32-key halves, each a full online-softmax step
  // (S_h = K_h Q^T, masked, exponentiated, O += V_h P_h); the running maximum moves only
  // when some row's grows by more than 2^kTau (decided per wave), and the accumulator is
  // then rescaled before the half's product is added.
  auto half_softmax = [&](f32x16& sc, int kvh, bool mask, bf16x8& p_lo, bf16x8& p_hi, float& alpha)
      __attribute__((always_inline)) -> bool {
    if (mask) {
      // register r holds key kvh + 8 (r / 4) + 4 hl + r % 4
      const int lim = q - kvh - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = (8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : sc[r];
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = max_across_halves(mx);
    const float mxs = mx * c2;
    const bool need = __any(mxs > m_run + kTau);
    const float m_use = need ? fmaxf(m_run, mxs) : m_run;
    alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_use;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -m_run));
    // P in bf16 (the MFMA operand); the row sum adds the same rounded values, so the
    // weights the output is normalised with are exactly the ones it was accumulated with
    u32x4 pw[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) pw[i >> 2][i & 3] = pack_bf16x2(sc[2 * i], sc[2 * i + 1]);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ls = add_bf16x2(pw[i >> 2][i & 3], ls);
    l_part = fmaf(l_part, alpha, ls);
    p_lo = as_bf16x8(pw[0]);
    p_hi = as_bf16x8(pw[1]);
    return need;
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
  };
  auto qk_half = [&](const uint16_t* kt, int half, f32x16& sc) __attribute__((always_inline)) {
    sc = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ak = as_bf16x8(ld16(kt + g_rd + half * 256 * CPR + 256 * ks));
      sc = mfma32x32x16(ak, as_bf16x8(qreg[ks]), sc);
    }
  };
  // k-steps j4 = 2 half + {0, 1} of the P V product take their keys from this half
  auto pv_half = [&](const uint16_t* kt, int half, const bf16x8& p_lo, const bf16x8& p_hi)
      __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint16_t* vp = kt + v_rd + 4 * (2 * half + jj) * 32 * CPR + 128 * db;
        const u32x2 v0 = lds_read_tr16(vp);
        const u32x2 v1 = lds_read_tr16(vp + 2 * 32 * CPR);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
        acc_o[db] = mfma32x32x16(av, jj ? p_hi : p_lo, acc_o[db]);
      }
  };
  // The mask test is a wave-uniform branch around the masking only: one copy of the tile
  // body, so the accumulators keep their registers on every path.
  auto tile_body = [&](const uint16_t* kt, int kv0, bool kMask) __attribute__((always_inline)) {
    f32x16 s0, s1;
    bf16x8 p0, p1, p2, p3;
    float a0, a1;
    qk_half(kt, 0, s0);
    const bool n0 = half_softmax(s0, kv0, kMask, p0, p1, a0);
    if (n0) rescale(a0);
    pv_half(kt, 0, p0, p1);
    qk_half(kt, 1, s1);
    const bool n1 = half_softmax(s1, kv0 + 32, kMask, p2, p3, a1);
    if (n1) rescale(a1);
    pv_half(kt, 1, p2, p3);
  };

  // iteration j: buffer j%2 holds tile j; tile j+1 (or M^T) is copied into the other one
  auto step = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* kt = bufp(bufc);
    uint16_t* other = bufp(IC<buf ^ 1>{});
    if (j + 1 < nkv) load_tile(j + 1, other);
    else load_mt(other);
    const int kv0 = j * kBN;
    if (kv0 <= qw0 + 31) {
      tile_body(kt, kv0, kv0 + kBN - 1 > qw0);   // mask when some keys lie past this wave's queries
    }
    __syncthreads();   // waits for this wave's copies, then for every wave's
  };
  for (int j = 0; j < nkv; j += 2) {
    step(j, IC<0>{});
    if (j + 1 < nkv) step(j + 1, IC<1>{});
  }

  // ---------------------------------------------------------------- epilogue
  // M^T_{s-1} is in buffer nkv % 2 (z_{s-1} in zsh); the output is staged in the other one
  const uint16_t* mts = (nkv & 1) ? buf1 : buf0;
  uint16_t* ost = ((nkv & 1) ? buf0 : buf1) + wave * 32 * D;
  const float l_tot = sum_across_halves(l_part);
  const float inv_l = 1.f / l_tot;

  // sigma(Q) as the B operand of the retrieval, and the denominator sigma(q) . z_{s-1}
  float den = 0.f;
  bf16x8 sq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(zsh + 16 * ks + 8 * hl);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(zsh + 16 * ks + 8 * hl + 4);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[2 * i] = elu_plus_one(bf16lo_to_f32(qreg[ks][i]));
      sv[2 * i + 1] = elu_plus_one(bf16hi_to_f32(qreg[ks][i]));
    }
    den += sv[0] * z0[0] + sv[1] * z0[1] + sv[2] * z0[2] + sv[3] * z0[3] +
           sv[4] * z1[0] + sv[5] * z1[1] + sv[6] * z1[2] + sv[7] * z1[3];
    sq[ks] = as_bf16x8(u32x4{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                             pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7])});
  }
  den = sum_across_halves(den);
  const float inv_den = 1.f / (den + a.eps);
  const float g = a.gate_g[h], omg = a.gate_omg[h];

#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 acc_m = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 am = as_bf16x8(ld16(mts + g_rd + db * 256 * CPR + 256 * ks));
      acc_m = mfma32x32x16(am, sq[ks], acc_m);
    }
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float amem = acc_m[r] * inv_den;
      const float adot = acc_o[db][r] * inv_l;
      o[r] = g * amem + omg * adot;
      if constexpr (PARTS) {
        if (q < n) {
          const int dv = 32 * db + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int64_t e = (row0 + q) * D + dv;
          if (a.a_mem) a.a_mem[e] = amem;
          if (a.a_dot) a.a_dot[e] = adot;
        }
      }
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      st8(ost + l32 * D + 8 * ((4 * db + r4) ^ swz(l32)) + 4 * hl,
          u32x2{pack_bf16x2(o[4 * r4], o[4 * r4 + 1]), pack_bf16x2(o[4 * r4 + 2], o[4 * r4 + 3])});
  }
  __syncthreads();
  uint16_t* og = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int i = 0; i < 32 * D / 8 / 64; ++i) {
    const int id = lane + 64 * i;
    const int row = id / (D / 8), c = id % (D / 8);
    if (qw0 + row < n) st16(og + (row0 + qw0 + row) * D + 8 * c, ld16(ost + row * D + 8 * (c ^ swz(row))));
  }
}

// ------------------------------------------------------------------ float32 I/O path
// Plain SIMT version for fp32 inputs and outputs: 64 queries per workgroup, TPR threads
// per query (32 head features each), per-key online softmax, fp32 everywhere.
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void k_attn_f32(const WindowArgs a) {
  constexpr int TPR = D / 32;
  constexpr int QB = 64;
  constexpr int KT = 32;
  __shared__ float ks_lds[KT][D];
  __shared__ float vs_lds[KT][D];
  __shared__ float sq_lds[QB][D];

  const int units = a.units();
  const int u = static_cast<int>(blockIdx.x) % units;
  const int qb = static_cast<int>(blockIdx.x) / units;
  const int BH = a.B * a.H;
  const int s_local = u / BH, bh = u % BH, h = bh % a.H;
  const int n = a.seg_tokens(s_local);
  const int q0 = qb * QB;
  if (q0 >= n) return;
  const int64_t row0 = static_cast<int64_t>(bh) * a.T + static_cast<int64_t>(a.s0 + s_local) * a.N;
  const int tid = threadIdx.x;
  const int qi = tid / TPR, part = tid % TPR;
  const int q = q0 + qi;
  const int d0 = part * 32;
  const float* qg = static_cast<const float*>(a.q);
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);

  float qv[32], o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    qv[i] = (q < n) ? qg[(row0 + q) * D + d0 + i] : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(q0 + QB, n);
  for (int t0 = 0; t0 < kv_end; t0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * D; e += blockDim.x) {
      const int t = e / D, d = e % D;
      const bool ok = t0 + t < n;
      ks_lds[t][d] = ok ? kg[(row0 + t0 + t) * D + d] : 0.f;
      vs_lds[t][d] = ok ? vg[(row0 + t0 + t) * D + d] : 0.f;
    }
    __syncthreads();
    for (int t = 0; t < KT; ++t) {
      const int kv = t0 + t;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) s += qv[i] * ks_lds[t][d0 + i];
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (kv > q || kv >= n) continue;   // uniform within the query's TPR group
      s *= a.scale;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float p = expf(s - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = o[i] * alpha + p * vs_lds[t][d0 + i];
      m = m_new;
    }
  }
  // retrieval: sigma(q) M_{s-1} / (sigma(q) z_{s-1} + eps), M^T stored [d_value][d_key]
  const float* mt = static_cast<const float*>(a.ws.mt) + static_cast<int64_t>(u) * D * D;
  const float* zb = a.ws.zb + static_cast<int64_t>(u) * D;
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float s = elu_plus_one(qv[i]);
    sq_lds[qi][d0 + i] = s;
    den += s * zb[d0 + i];
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  __syncthreads();
  const float inv_den = 1.f / (den + a.eps);
  const float g = a.gate_g[h], omg = a.gate_omg[h];
  float* og = static_cast<float*>(a.out);
  for (int i = 0; i < 32; ++i) {
    const int dv = d0 + i;
    float num = 0.f;
    for (int k = 0; k < D; ++k) num += sq_lds[qi][k] * mt[static_cast<int64_t>(dv) * D + k];
    const float amem = num * inv_den;
    const float adot = o[i] / l;
    if (q < n) {
      const int64_t e = (row0 + q) * D + dv;
      og[e] = g * amem + omg * adot;
      if (a.a_mem) a.a_mem[e] = amem;
      if (a.a_dot) a.a_dot[e] = adot;
    }
  }
}

template <int D>
hipError_t launch_attention_d(const WindowArgs& a, hipStream_t st) {
  if (a.bf16) {
    const dim3 grid(a.units() * ((a.N + kBM - 1) / kBM));
    if (a.a_mem || a.a_dot) hipLaunchKernelGGL((k_attn_bf16<D, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_attn_bf16<D, false>), grid, dim3(kThreads), 0, st, a);
  } else {
    const dim3 grid(a.units() * ((a.N + 63) / 64));
    hipLaunchKernelGGL((k_attn_f32<D>), grid, dim3(64 * (D / 32)), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const WindowArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_attention_d<128>(a, st) : launch_attention_d<64>(a, st);
}

}  // namespace infini
