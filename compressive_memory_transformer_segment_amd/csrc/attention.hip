// Fused per-segment output of the Infini-attention layer (architecture summary of
// arXiv 2404.07143, section 3.4):
//
//   A_dot = softmax(scale * Q K^T, causal inside the segment) V                  (Eq. 6)
//   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)                          (Eq. 7)
//   out   = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot                   (Eq. 10)
//
// bf16 path: one workgroup = 8 waves = 256 queries of one (batch, head, segment); every
// wave owns 32 queries.  The kernel works in the transposed frame: S^T = K Q^T and O^T = V^T P^T, so
// that a lane holds one query (lane % 32) in every MFMA result.  Softmax statistics are
// then per-lane scalars (plus one exchange with lane ^ 32), the S^T result registers are
// directly the B operand of O^T += V^T P^T, and the retrieval sigma(Q) reuses the Q
// registers (Q is the B operand of S^T) as the B operand of A_mem^T = M^T sigma(Q)^T.
//
// K and V tiles (64 keys x d) go from HBM straight into LDS with buffer -> LDS copies,
// four buffers deep: the copy of tile j + 3 (after the last tile: M^T_{s-1} and z_{s-1})
// is in flight while tile j is consumed, and no registers hold data in transit.  The
// scores of tile j + 1 are computed while the softmax of tile j runs, and every group of
// MFMAs finds its LDS operands already read into registers.  Rows past the segment end
// arrive as zeros (buffer range check), so ragged tails need no branches.
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

constexpr int kThreadsA = 512;   // bf16 path: 8 waves
constexpr int kBMA = 256;        // bf16 path: queries per workgroup (8 waves x 32)
constexpr int kBN = 64;          // keys per tile
constexpr float kTau = 8.f;

template <int N_>
using IC = std::integral_constant<int, N_>;

// Workgroup -> (unit, query tile).  Workgroups are dispatched to the 8 XCDs round-robin
// (block b to XCD b % 8), and each XCD has its own L2.  When the unit count is a multiple
// of 8, XCD x takes the units u = x + 8 k in groups of kGroup units; inside a group the
// query tiles run longest first.  About kGroup units' K and V are then live in one L2 at
// a time, and the short diagonal tiles of each group fill in behind the long ones.
// Otherwise: longest tiles first across all units.
constexpr int kGroup = 4;
template <int BM>
__device__ __forceinline__ void tile_of_block(int units, int nq, int& u, int& qt) {
  const int b = static_cast<int>(blockIdx.x);
  if (units % 8 != 0) {
    qt = nq - 1 - b / units;
    u = b % units;
    return;
  }
  const int x = b % 8, i = b / 8;            // XCD and position in its sequence
  const int per_x = units / 8;               // units of this XCD
  const int gi = i / (kGroup * nq);          // group index
  const int g_units = min(kGroup, per_x - gi * kGroup);
  const int r = i - gi * kGroup * nq;        // position inside the group
  qt = nq - 1 - r / g_units;
  u = x + 8 * (gi * kGroup + r % g_units);
}

// MODE: 0 = the gated output; 1 = also A_mem, A_dot (fp32) and the log-sum-exp; 2 = the
// backward's per-token terms instead of the output: log-sum-exp, D = dO . A_dot, the
// retrieval denominator, its gradient -g dO . A_mem / den, and the gate term
// g (1 - g) dO . (A_mem - A_dot) (dO given in bwd_dout).
template <int D, int MODE>
__global__ __launch_bounds__(kThreadsA, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(const WindowArgs a) {
  constexpr int KS = D / 16;                  // k-steps over the head dimension
  constexpr int DB = D / 32;                  // 32-row blocks of the head dimension
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = kBN * D;               // elements of one K or V tile
  constexpr int BUF = 2 * TILE;               // one buffer: [K tile | V tile]
  constexpr int CW = CPR / 8;                 // 1 KB copies per wave for a K (or V) tile
  constexpr int MW = D * D / 4096;            // ... for M^T_{s-1}
  static_assert(D * D <= BUF && 4 * 32 * D <= BUF, "M^T and four waves' output fit in one buffer");

  // LDS layouts (bf16, 16-byte chunks; chunk c of a row holds columns 8c .. 8c + 7):
  //  "row groups" for K and M^T: chunk c of row r sits in slot (r / 16) * 16 CPR + 16 c + r % 16,
  //  so the 16 rows an MFMA operand read touches at one chunk are 16 consecutive slots
  //  (one 256-byte bank line), and every k-step / row block is an immediate offset;
  //  "quads" for V: chunk c of row r sits in slot (r / 4) * 4 CPR + 4 c + r % 4, so the
  //  4 rows x 64 bytes a transpose read takes per half-wave are 16 consecutive slots.
  // Both are filled by 1 KB buffer -> LDS copies (64 lanes x 16 bytes, lane i to slot
  // 64 c + i of copy c); what differs between a wave's copies sits in the scalar resource
  // base and the LDS base, so one offset register per layout suffices.
  // Four buffers: the copy of tile j + 3 (then M^T_{s-1}) is in flight while tile j is
  // consumed.  After the loop the output is staged row-major, chunk c of row r at
  // physical chunk c ^ swz(r), in two of the free buffers.
  __shared__ __align__(16) uint16_t buf0[BUF];
  __shared__ __align__(16) uint16_t buf1[BUF];
  __shared__ __align__(16) uint16_t buf2[BUF];
  __shared__ __align__(16) uint16_t buf3[BUF];
  __shared__ __align__(16) float zsh[256];

  const int units = a.units();
  const int nq = (a.N + kBMA - 1) / kBMA;
  int u, qt;
  tile_of_block<kBMA>(units, nq, u, qt);
  const int BH = a.B * a.H;
  const int s_local = u / BH, bh = u % BH, h = bh % a.H;
  const int n = a.seg_tokens(s_local);
  const int q0 = qt * kBMA;
  if (q0 >= n) return;
  const int64_t tok0 = static_cast<int64_t>(a.s0 + s_local) * a.N;
  const int64_t row0 = static_cast<int64_t>(bh) * a.T + tok0;   // token row of the segment start

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, 0 .. 7
  const int l32 = lane & 31, hl = lane >> 5;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + l32;

  // Q and K of the local attention (position-embedded when the caller supplies them)
  const uint16_t* qg = static_cast<const uint16_t*>(a.q_loc) + row0 * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k_loc) + row0 * D;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + row0 * D;

  u32x4 qreg[KS];   // Q as the B operand of S^T: lane holds Q[q][16 ks + 8 hl .. +7]

  // source byte offsets of this lane's 16 bytes within a copy:
  //   row groups, copy c = (CPR / 4) g + j: row 16 g + lane % 16, chunk 4 j + lane / 16
  //   quads, copy c: row 4 (CPR c / 16 + lane / (4 CPR)) + lane % 4, chunk (lane / 4) % CPR
  const uint32_t lp_g = (lane & 15) * (2 * D) + 16 * (lane >> 4);
  const uint32_t lp_v = (((lane >> 2) / CPR) * 4 + (lane & 3)) * (2 * D) + 16 * ((lane >> 2) % CPR);
  // one copy: the resource starts `shift` bytes into the source (bytes past `bytes` of the
  // source read as zeros), the 1 KB lands at lds
  auto copy1k = [&](const void* src, uint32_t bytes, uint32_t shift, void* lds, uint32_t voff)
      __attribute__((always_inline)) {
    const int left = __builtin_amdgcn_readfirstlane(max(static_cast<int>(bytes) - static_cast<int>(shift), 0));
    buffer_to_lds16(buffer_rsrc(static_cast<const char*>(src) + shift, static_cast<uint32_t>(left)), lds, voff);
  };
  auto copy_group = [&](int c, const void* src, uint32_t bytes, uint16_t* dst) __attribute__((always_inline)) {
    const int g = c / (CPR / 4), j = c % (CPR / 4);
    copy1k(src, bytes, g * 32 * D + 64 * j, reinterpret_cast<char*>(dst) + c * 1024, lp_g);
  };
  auto bufp = [&](auto bc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int b = decltype(bc)::value & 3;
    if constexpr (b == 0) return buf0;
    else if constexpr (b == 1) return buf1;
    else if constexpr (b == 2) return buf2;
    else return buf3;
  };
  const int nkv = (min(q0 + kBMA, n) + kBN - 1) / kBN;
  // Copy number i of the sequence: K and V of tile i for i < nkv (rows at or past the
  // segment end arrive as zeros), M^T_{s-1} and z_{s-1} for i == nkv, nothing after.
  // Returns how many copy instructions this wave issued.
  auto issue = [&](int i, uint16_t* dst) __attribute__((always_inline)) -> int {
    if (i < nkv) {
      const int kv0 = i * kBN;
      const uint32_t bytes = static_cast<uint32_t>(n - kv0) * D * 2;
      const uint16_t* ksrc = kg + static_cast<int64_t>(kv0) * D;
      const uint16_t* vsrc = vg + static_cast<int64_t>(kv0) * D;
#pragma unroll
      for (int t = 0; t < CW; ++t) copy_group(wave * CW + t, ksrc, bytes, dst);
#pragma unroll
      for (int t = 0; t < CW; ++t) {
        const int c = wave * CW + t;
        copy1k(vsrc, bytes, 1024 * c, reinterpret_cast<char*>(dst + TILE) + 1024 * c, lp_v);
      }
      return 2 * CW;
    }
    if (i == nkv) {
      const uint16_t* msrc = static_cast<const uint16_t*>(a.ws.mt) + static_cast<int64_t>(u) * D * D;
#pragma unroll
      for (int t = 0; t < MW; ++t) copy_group(wave * MW + t, msrc, D * D * 2, dst);
      if (wave == 0) {   // lanes past D / 4 read zeros
        copy1k(a.ws.zb + static_cast<int64_t>(u) * D, D * 4, 0, zsh, static_cast<uint32_t>(lane) * 16);
        return MW + 1;
      }
      return MW;
    }
    return 0;
  };
  auto count = [&](int i) __attribute__((always_inline)) -> int {
    return i < nkv ? 2 * CW : (i == nkv ? MW + (wave == 0 ? 1 : 0) : 0);
  };

  // element offsets of this lane's operand reads
  //  K / M^T (row groups): row 32 blk + l32, chunk 2 ks + hl -> g_rd + blk * 256 CPR + ks * 256
  //  V^T (quads, transpose reads): k-slot (hl, i) of k-step j4 is key
  //    16 j4 + 8 (i / 4) + 4 hl + i % 4, the key the S^T register feeding that slot holds;
  //    the lane addresses row 16 j4 + 8 s + 4 hl + (lane % 16) / 4 and columns
  //    32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. +3
  //    -> v_rd + (4 j4 + 2 s) * 32 CPR + db * 128
  const int g_rd = ((l32 >> 4) * 16 * CPR + 16 * hl + (l32 & 15)) * 8;
  const int v_rd = TILE + (hl * 4 * CPR + (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * 4 + ((lane & 15) >> 2)) * 8 +
                   4 * (lane & 1);
  auto swz = [](int row) __attribute__((always_inline)) -> int { return D == 128 ? (row & 15) : ((row >> 1) & 7); };

  // ---- prologue.  Every lane loads its query's Q row straight into the B-operand
  // registers (rows >= n read as zeros); tiles 0, 1 and 2 go into buffers 0, 1 and 2.
  {
    const auto qr = buffer_rsrc(qg + static_cast<int64_t>(qw0) * D, static_cast<uint32_t>(max(n - qw0, 0)) * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = buffer_ld16(qr, static_cast<uint32_t>(l32 * D + 16 * ks + 8 * hl) * 2);
    issue(0, buf0);
    issue(1, buf1);
    issue(2, buf2);
    wait_vm_le(0);
    __builtin_amdgcn_s_barrier();
  }

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;   // running row maximum, scaled (log2 domain)
  float l_part = 0.f;        // this lane's half of the row sum
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = zero16();

  // Online softmax, one decision per 64-key tile: the running maximum m_run (log2 domain,
  // scale folded in) moves only when some row's maximum over the tile exceeds it by more
  // than kTau (decided per wave); O and the row sum are then rescaled once, before any of
  // the tile's products.  Otherwise the tile is straight-line code.
  auto mask_half = [&](f32x16& sc, int kvh) __attribute__((always_inline)) {
    // register r holds key kvh + 8 (r / 4) + 4 hl + r % 4
    const int lim = q - kvh - 4 * hl;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = (8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : sc[r];
  };
  auto half_max = [&](const f32x16& sc) __attribute__((always_inline)) -> float {
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    return mx;
  };
  // P = exp2(scale log2e S - m_run) in bf16 (the MFMA operand); the row sum adds the same
  // rounded values, so the output is normalised with exactly the weights it accumulated
  auto half_exp = [&](f32x16& sc, bf16x8& p_lo, bf16x8& p_hi) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -m_run));
    u32x4 pw[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) pw[i >> 2][i & 3] = pack_bf16x2(sc[2 * i], sc[2 * i + 1]);
    float ls = l_part;
#pragma unroll
    for (int i = 0; i < 8; ++i) ls = add_bf16x2(pw[i >> 2][i & 3], ls);
    l_part = ls;
    p_lo = as_bf16x8(pw[0]);
    p_hi = as_bf16x8(pw[1]);
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
  };
  // S^T of both halves: all 2 KS K-operand reads are issued first (their LDS latency then
  // overlaps), and the two accumulation chains alternate so that consecutive MFMAs are
  // independent.
  auto qk_tile = [&](const uint16_t* kt, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    bf16x8 ak[2][KS];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ak[hh][ks] = as_bf16x8(ld16(kt + g_rd + hh * 256 * CPR + 256 * ks));
    __builtin_amdgcn_sched_barrier(0);
    s0 = zero16();
    s1 = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32x32x16(ak[0][ks], as_bf16x8(qreg[ks]), s0);
      s1 = mfma32x32x16(ak[1][ks], as_bf16x8(qreg[ks]), s1);
    }
  };
  // V^T operands of one half (k-steps j4 = 2 half + {0, 1} take their keys from it)
  auto v_operands = [&](const uint16_t* kt, int half, bf16x8 (&av)[DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint16_t* vp = kt + v_rd + 4 * (2 * half + jj) * 32 * CPR + 128 * db;
        const u32x2 v0 = lds_read_tr16(vp);
        const u32x2 v1 = lds_read_tr16(vp + 2 * 32 * CPR);
        av[db][jj] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
      }
  };
  auto pv = [&](const bf16x8 (&av)[DB][2], const bf16x8& p_lo, const bf16x8& p_hi) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] = mfma32x32x16(av[db][jj], jj ? p_hi : p_lo, acc_o[db]);
  };
  auto tile_max = [&](const f32x16& s0, const f32x16& s1) __attribute__((always_inline)) -> float {
    return max_across_halves(fmaxf(half_max(s0), half_max(s1))) * c2;
  };
  auto maybe_rescale = [&](float mxs) __attribute__((always_inline)) {
    if (__any(mxs > m_run + kTau)) {
      const float m_use = fmaxf(m_run, mxs);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      rescale(alpha);
      l_part *= alpha;
      m_run = m_use;
    }
  };
  // P_A, O += V_A P_A, P_B, O += V_B P_B for a tile whose scores are in s0 / s1.  The V^T
  // reads of a half are issued before its exponentials, which cover their latency; the
  // exponentials of B run under the MFMAs of A.
  auto finish_tile = [&](const uint16_t* kt, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    bf16x8 p0, p1, p2, p3;
    bf16x8 va[DB][2], vb[DB][2];
    v_operands(kt, 0, va);
    half_exp(s0, p0, p1);
    v_operands(kt, 1, vb);
    pv(va, p0, p1);
    half_exp(s1, p2, p3);
    pv(vb, p2, p3);
  };

  // Unmasked tiles j < jm = q0 / 64 (a multiple of 4) run software-pipelined: iteration j
  // holds the scores of tile j (sc0 / sc1, maximum mxc) and computes those of tile j + 1
  // while it exponentiates and multiplies tile j, so a wave's own MFMAs run under its
  // softmax arithmetic.  Every group of MFMAs finds its LDS operands already in registers:
  // the operands of the next group are read while a group runs.  An iteration has four
  // phases of 8 MFMAs each:
  //   1. S^T(j + 1), k-steps 0 .. KS/2 - 1 (both key halves) | exp of tile j, half 0 | read K, k-steps KS/2 ..
  //   2. S^T(j + 1), k-steps KS/2 .. KS - 1                 | exp of tile j, half 1 | read V^T(j), half 0
  //   3. O^T += V^T P^T(j), half 0                          | max of tile j + 1    | read V^T(j), half 1
  //   4. O^T += V^T P^T(j), half 1                          |                      | read K(j + 2), k-steps 0 ..
  // Buffer j % 4 holds tile j.  Copy j + 3 of the sequence is issued at the start of
  // iteration j into buffer (j + 3) % 4 (tile j - 1, done with at the previous barrier) and
  // waited for at its end, so tiles j + 1 and j + 2 are complete throughout iteration j.
  const int jm = q0 / kBN;
  constexpr int KH = KS / 2;   // k-steps per operand group
  typedef bf16x8 KOps[2][KH];  // [key half][k-step]
  auto load_k = [&](const uint16_t* kt, int k0, KOps& ak) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < KH; ++i) ak[hh][i] = as_bf16x8(ld16(kt + g_rd + hh * 256 * CPR + 256 * (k0 + i)));
  };
  auto qk_part = [&](const KOps& ak, int k0, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KH; ++i) {
      s0 = mfma32x32x16(ak[0][i], as_bf16x8(qreg[k0 + i]), s0);
      s1 = mfma32x32x16(ak[1][i], as_bf16x8(qreg[k0 + i]), s1);
    }
  };
  f32x16 sc0, sc1;
  KOps kq;
  load_k(buf0, 0, kq);
  sc0 = zero16();
  sc1 = zero16();
  qk_part(kq, 0, sc0, sc1);
  load_k(buf0, KH, kq);
  qk_part(kq, KH, sc0, sc1);   // tile 0
  float mxc = tile_max(sc0, sc1);
  if (jm > 0) load_k(buf1, 0, kq);   // tile 1, k-steps 0 .. KH - 1
  auto pstep = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    maybe_rescale(mxc);
    issue(j + 3, bufp(IC<b + 3>{}));
    const uint16_t* kt = bufp(bufc);
    f32x16 n0 = zero16(), n1 = zero16();
    bf16x8 p0, p1, p2, p3;
    KOps kq2;
    bf16x8 va[DB][2], vb[DB][2];
    // phase 1
    load_k(bufp(IC<b + 1>{}), KH, kq2);
    qk_part(kq, 0, n0, n1);
    half_exp(sc0, p0, p1);
    // interleave: each MFMA followed by its share of the LDS reads and the VALU work
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 48 / KS, 0);   // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 2
    v_operands(kt, 0, va);
    qk_part(kq2, KH, n0, n1);
    half_exp(sc1, p2, p3);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB / KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 48 / KS, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 3
    v_operands(kt, 1, vb);
    pv(va, p0, p1);
    const float mh0 = half_max(n0);
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 4
    load_k(bufp(IC<b + 2>{}), 0, kq);   // tile j + 2 (read but unused past the last tile)
    pv(vb, p2, p3);
    mxc = max_across_halves(fmaxf(mh0, half_max(n1))) * c2;
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, KS / DB, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    sc0 = n0;
    sc1 = n1;
    wait_vm_le(0);
    __builtin_amdgcn_s_barrier();
  };
  for (int j = 0; j < jm; j += 4) {
    pstep(j, IC<0>{});
    pstep(j + 1, IC<1>{});
    pstep(j + 2, IC<2>{});
    pstep(j + 3, IC<3>{});
  }
  // The (up to) four tiles from q0 on hold the diagonal of every wave: masked, one at a
  // time; tile jm's scores are already in sc0 / sc1.  A wave skips a tile whose keys all
  // lie past its queries.
  auto mstep = [&](int j, auto bufc, bool have_scores) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    const uint16_t* kt = bufp(bufc);
    issue(j + 3, bufp(IC<b + 3>{}));
    const int kv0 = j * kBN;
    if (kv0 <= qw0 + 31) {
      if (!have_scores) qk_tile(kt, sc0, sc1);
      mask_half(sc0, kv0);
      mask_half(sc1, kv0 + 32);
      maybe_rescale(tile_max(sc0, sc1));
      finish_tile(kt, sc0, sc1);
    }
    wait_vm_le(count(j + 2) + count(j + 3));
    __builtin_amdgcn_s_barrier();
  };
  mstep(jm, IC<0>{}, true);
  if (jm + 1 < nkv) mstep(jm + 1, IC<1>{}, false);
  if (jm + 2 < nkv) mstep(jm + 2, IC<2>{}, false);
  if (jm + 3 < nkv) mstep(jm + 3, IC<3>{}, false);
  wait_vm_le(0);   // M^T_{s-1} and z_{s-1}
  __builtin_amdgcn_s_barrier();

  // ---------------------------------------------------------------- epilogue
  // M^T_{s-1} is in buffer nkv % 4 (z_{s-1} in zsh); the output is staged in buffers
  // (nkv + 1) % 4 (waves 0-3) and (nkv + 2) % 4 (waves 4-7)
  auto buf_at = [&](int i) __attribute__((always_inline)) -> uint16_t* {
    switch (i & 3) {
      case 0: return buf0;
      case 1: return buf1;
      case 2: return buf2;
      default: return buf3;
    }
  };
  const uint16_t* mts = buf_at(nkv);
  uint16_t* ost = buf_at(nkv + 1 + (wave >> 2)) + (wave & 3) * 32 * D;
  const float l_tot = sum_across_halves(l_part);
  const float inv_l = 1.f / l_tot;
  if constexpr (MODE >= 1) {
    if (a.lse && hl == 0 && q < n) a.lse[row0 + q] = m_run + __log2f(l_tot);
  }

  // With a separate local Q the retrieval needs the PE-free Q rows: each wave copies its
  // own 32 rows into its (not yet used) staging region and reads them back, as in the
  // prologue.
  if (a.q_loc != a.q) {
    const uint16_t* qm = static_cast<const uint16_t*>(a.q) + (row0 + qw0) * D;
    const uint32_t qbytes = static_cast<uint32_t>(max(n - qw0, 0)) * D * 2;
#pragma unroll
    for (int c = 0; c < CPR / 2; ++c) copy_group(c, qm, qbytes, ost);
    wait_vm_le(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = ld16(ost + g_rd + 256 * ks);
    wait_vm_le(0);   // the reads are done before the region is reused for the output
  }

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
  float ddp = 0.f, emp = 0.f;   // MODE 2: this lane's shares of dO . A_dot and dO . A_mem
  const uint16_t* dog = MODE == 2 ? static_cast<const uint16_t*>(a.bwd_dout) + (row0 + q) * D : nullptr;

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
      if constexpr (MODE == 1) {
        if (q < n) {
          const int dv = 32 * db + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int64_t e = (row0 + q) * D + dv;
          if (a.a_mem) a.a_mem[e] = amem;
          if (a.a_dot) a.a_dot[e] = adot;
        }
      }
    }
    if constexpr (MODE == 2) {
      if (q < n) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2 dv = ld8(dog + 32 * db + 8 * r4 + 4 * hl);
          const float df[4] = {bf16lo_to_f32(dv[0]), bf16hi_to_f32(dv[0]), bf16lo_to_f32(dv[1]), bf16hi_to_f32(dv[1])};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ddp = fmaf(df[e], acc_o[db][4 * r4 + e] * inv_l, ddp);
            emp = fmaf(df[e], acc_m[4 * r4 + e] * inv_den, emp);
          }
        }
      }
    } else {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        st8(ost + l32 * D + 8 * ((4 * db + r4) ^ swz(l32)) + 4 * hl,
            u32x2{pack_bf16x2(o[4 * r4], o[4 * r4 + 1]), pack_bf16x2(o[4 * r4 + 2], o[4 * r4 + 3])});
    }
  }
  if constexpr (MODE == 2) {
    ddp = sum_across_halves(ddp);
    emp = sum_across_halves(emp);
    if (hl == 0 && q < n) {
      const int64_t rq = row0 + q;
      const float dn = den + a.eps;
      a.bwd_dd[rq] = ddp;
      a.bwd_den[rq] = dn;
      a.bwd_dden[rq] = -g * emp / dn;
      a.bwd_bq[rq] = (emp - ddp) * g * omg;
    }
    return;
  }
  // each wave reads back only the rows it staged
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  const float* qg = static_cast<const float*>(a.q_loc);   // local attention's Q and K
  const float* kg = static_cast<const float*>(a.k_loc);
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
  if (a.q_loc != a.q) {   // the retrieval reads the PE-free Q
    const float* qm = static_cast<const float*>(a.q);
#pragma unroll
    for (int i = 0; i < 32; ++i) qv[i] = (q < n) ? qm[(row0 + q) * D + d0 + i] : 0.f;
  }
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
  // natural-log softmax state -> the log2 domain of the bf16 path
  if (a.lse && part == 0 && q < n) a.lse[row0 + q] = (m + __logf(l)) * kLog2e;
}

template <int D>
hipError_t launch_attention_d(const WindowArgs& a, hipStream_t st) {
  if (a.bf16) {
    const dim3 grid(a.units() * ((a.N + kBMA - 1) / kBMA));
    if (a.bwd_dout) hipLaunchKernelGGL((k_attn_bf16<D, 2>), grid, dim3(kThreadsA), 0, st, a);
    else if (a.a_mem || a.a_dot || a.lse) hipLaunchKernelGGL((k_attn_bf16<D, 1>), grid, dim3(kThreadsA), 0, st, a);
    else hipLaunchKernelGGL((k_attn_bf16<D, 0>), grid, dim3(kThreadsA), 0, st, a);
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
