// Fused per-segment output of the Infini-attention layer (architecture summary of
// arXiv 2404.07143, section 3.4):
//
//   A_dot = softmax(scale * Q K^T, causal inside the segment) V                  (Eq. 6)
//   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)                          (Eq. 7)
//   out   = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot                   (Eq. 10)
//
// bf16 path: a persistent grid of at most one workgroup per compute unit; a workgroup
// (8 waves) walks a sequence of items, an item being 256 queries of one (batch, head,
// segment), and every wave owns 32 queries of it.  The kernel works in the transposed
// frame: S^T = K Q^T and O^T = V^T P^T, so that a lane holds one query (lane % 32) in
// every MFMA result.  Softmax statistics are then per-lane scalars (plus one exchange with
// lane ^ 32), the S^T result registers are directly the B operand of O^T += V^T P^T, and
// the retrieval sigma(Q) reuses the Q registers (Q is the B operand of S^T) as the B
// operand of A_mem^T = M^T sigma(Q)^T.
//
// K and V tiles (64 keys x d) go from HBM straight into LDS with buffer -> LDS copies, in
// a ring of four buffers: the copy of tile j + 3 is in flight while tile j is consumed,
// and no registers hold data in transit.  The ring runs on across items: the last steps of
// an item fetch the next item's first three tiles, and its epilogue the next item's Q
// rows.  M^T_{s-1} has a fifth buffer of its own.  The scores of tile j + 1 are computed
// while the softmax of tile j runs, and every group of MFMAs finds its LDS operands
// already read into registers.  Rows past the segment end arrive as zeros (buffer range
// check), so ragged tails need no branches.
// The V^T operand of O^T += V^T P^T is read with LDS transpose reads, in the key order the
// S^T result registers hold.  The online softmax is in the exp2 domain with the scale
// folded in, and rescales the accumulator lazily: only when a row maximum grows by more
// than 2^8 (exact: the final division uses the same stale maximum).  The gated result
// goes from registers to memory: a swap between the two lane halves turns each lane's
// pieces of a row into whole 16-byte chunks.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kThreadsA = 512;   // bf16 path: 8 waves
constexpr int kBMA = 256;        // bf16 path: queries per workgroup (8 waves x 32)
constexpr int kBN = 64;          // keys per tile
constexpr float kTau = 8.f;
constexpr int kMaxChunks = 8;    // split mode: key chunks per query tile at most

template <int N_>
using IC = std::integral_constant<int, N_>;

// Persistent schedule.  The grid holds at most one workgroup per compute unit; each
// workgroup walks a sequence of items (unit, query tile), so that the first K / V tiles
// and the Q rows of its next item are fetched while the current one finishes.
// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b on XCD b % 8), and each
// XCD has its own L2.  When the unit count and the grid are multiples of 8, XCD x owns the
// units u = x + 8 k and orders their items in groups of kGroup units, longest query tiles
// first inside a group, so that about kGroup units' K and V are live in one L2 at a time.
// Round r gives the r-th slice of that order to the XCD's workgroups, in alternating
// direction (a workgroup that drew a long tile draws a short one next), which evens out
// the work per workgroup.  Otherwise the order is longest tiles first across all units.
constexpr int kGroup = 4;

// Division by a divisor fixed for the launch, for dividends below 2^31 (round-up method of
// Granlund and Montgomery, "Division by invariant integers using multiplication", 1994):
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1, a / d = (mulhi(a, m) + a) >> s.
// Scalar code on the GPU has no divide instruction; this is two operations.
struct FastDiv {
  uint32_t d = 1, m = 1, s = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t dd) : d(dd < 1 ? 1 : dd) {
    while ((uint64_t{1} << s) < d) ++s;
    m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << s) - d)) / d + 1);
  }
  __device__ __forceinline__ int div(int a) const {
    const uint32_t ua = static_cast<uint32_t>(a);
    return static_cast<int>((__umulhi(ua, m) + ua) >> s);
  }
  __device__ __forceinline__ int mod(int a) const { return a - div(a) * static_cast<int>(d); }
};
// The launch's divisors: units, kGroup x query tiles, the last group's unit count,
// B x H and H.
struct Sched {
  FastDiv units, grp, last, bh, h;
  FastDiv kc;   // split mode: key tiles per chunk
  int items;    // split mode: items per (batch, head) pair
};

__device__ __forceinline__ bool item_at(const Sched& sd, int units, int nq, int G, int r, int& u, int& qt) {
  const int b = static_cast<int>(blockIdx.x);
  if (units % 8 != 0 || G % 8 != 0) {
    const int i = r * G + ((r & 1) ? G - 1 - b : b);
    if (i >= units * nq) return false;
    const int iu = sd.units.div(i);
    qt = nq - 1 - iu;
    u = i - iu * units;
    return true;
  }
  const int x = b % 8, s = b / 8, gx = G / 8;   // XCD, slot on it, workgroups per XCD
  const int i = r * gx + ((r & 1) ? gx - 1 - s : s);   // position in the XCD's order
  const int per_x = units / 8;                          // units of this XCD
  if (i >= per_x * nq) return false;
  const int gi = sd.grp.div(i);                         // group index
  const int rr = i - gi * kGroup * nq;                  // position inside the group
  int qi, ui;                                           // rr / units in the group, rr % ...
  if (per_x - gi * kGroup >= kGroup) {
    qi = rr / kGroup;
    ui = rr % kGroup;
  } else {
    qi = sd.last.div(rr);
    ui = rr - qi * static_cast<int>(sd.last.d);
  }
  qt = nq - 1 - qi;
  u = x + 8 * (gi * kGroup + ui);
  return true;
}

// Split mode (one segment): item i = k * units + u, where k ranks the pair's items --
// query tiles from the last one down, and the key chunks of each in order (longest query
// tiles, whose chunks are all full, first).  Chunk c of query tile qt holds key tiles
// [c kc, min((c + 1) kc, nkv)).
__device__ __forceinline__ bool split_item_at(const Sched& sd, int units, int n, int G, int r, int& u, int& qt,
                                              int& c) {
  const int b = static_cast<int>(blockIdx.x);
  const int i = r * G + ((r & 1) ? G - 1 - b : b);
  if (i >= units * sd.items) return false;
  int k = sd.units.div(i);
  u = i - k * units;
  const int kc = static_cast<int>(sd.kc.d);
  for (int t = (n + kBMA - 1) / kBMA - 1; t >= 0; --t) {
    const int nkv = (min(t * kBMA + kBMA, n) + kBN - 1) / kBN;
    const int nc = sd.kc.div(nkv + kc - 1);
    if (k < nc) {
      qt = t;
      c = k;
      return true;
    }
    k -= nc;
  }
  return false;
}

// MODE: 0 = the gated output; 1 = also A_mem, A_dot (fp32) and the log-sum-exp; 2 = the
// backward's per-token terms instead of the output: log-sum-exp, D = dO . A_dot, the
// retrieval denominator, its gradient -g dO . A_mem / den, and the gate term
// g (1 - g) dO . (A_mem - A_dot) (dO given in bwd_dout).
// SPLIT: split-key mode (MODE 0 only): an item is one key chunk of a query tile; a query
// tile split into several chunks is finished by the workgroup whose chunk completes last.
template <int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(kThreadsA, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(const WindowArgs a, const Sched sd) {
  static_assert(!SPLIT || MODE == 0, "split-key mode writes the gated output only");
  constexpr int KS = D / 16;                  // k-steps over the head dimension
  constexpr int DB = D / 32;                  // 32-row blocks of the head dimension
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = kBN * D;               // elements of one K or V tile
  constexpr int BUF = 2 * TILE;               // one buffer: [K tile | V tile]
  constexpr int CW = CPR / 8;                 // 1 KB copies per wave for a K (or V) tile
  constexpr int MW = D * D / 4096;            // ... for M^T_{s-1}
  static_assert(D * D <= BUF, "M^T fits in one buffer");

  // LDS layouts (bf16, 16-byte chunks; chunk c of a row holds columns 8c .. 8c + 7):
  //  "row groups" for K and M^T: chunk c of row r sits in slot (r / 16) * 16 CPR + 16 c + r % 16,
  //  so the 16 rows an MFMA operand read touches at one chunk are 16 consecutive slots
  //  (one 256-byte bank line), and every k-step / row block is an immediate offset;
  //  "quads" for V: chunk c of row r sits in slot (r / 4) * 4 CPR + 4 c + r % 4, so the
  //  4 rows x 64 bytes a transpose read takes per half-wave are 16 consecutive slots.
  // Both are filled by 1 KB buffer -> LDS copies (64 lanes x 16 bytes, lane i to slot
  // 64 c + i of copy c); what differs between a wave's copies sits in the scalar resource
  // base and the LDS base, so one offset register per layout suffices.
  // Four K / V buffers in a ring (the copy of tile j + 3 is in flight while tile j is
  // consumed; the ring runs on into the next item) and one for M^T_{s-1}.
  __shared__ __align__(16) uint16_t buf0[BUF];
  __shared__ __align__(16) uint16_t buf1[BUF];
  __shared__ __align__(16) uint16_t buf2[BUF];
  __shared__ __align__(16) uint16_t buf3[BUF];
  __shared__ __align__(16) uint16_t bufm[D * D];

  const int units = a.units();
  const int nq = (a.N + kBMA - 1) / kBMA;
  const int G = static_cast<int>(gridDim.x);
  const int BH = a.B * a.H;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, 0 .. 7
  const int l32 = lane & 31, hl = lane >> 5;
  // Query block of this wave in an item: queries 32 qb .. 32 qb + 31.  Outside the split-key
  // mode the waves run the diagonal tiles each on its own, and waves w and w + 4 (one SIMD)
  // take blocks w and 7 - w, so that every SIMD has the same diagonal work (block b needs
  // diagonal key tiles 0 .. b / 2).
  constexpr bool kFree = !SPLIT;
  const int qb = kFree ? (wave < 4 ? wave : 11 - wave) : wave;

  // the next item of this workgroup at or after round r whose query tile holds tokens
  auto find = [&](int& r, int& u_, int& qt_, int& n_, int& c_) __attribute__((always_inline)) -> bool {
    if constexpr (SPLIT) {
      n_ = a.seg_tokens(0);
      return split_item_at(sd, units, n_, G, r, u_, qt_, c_);
    } else {
      c_ = 0;
      while (item_at(sd, units, nq, G, r, u_, qt_)) {
        n_ = a.seg_tokens(sd.bh.div(u_));
        if (qt_ * kBMA < n_) return true;
        ++r;
      }
      return false;
    }
  };
  const int kc = SPLIT ? static_cast<int>(sd.kc.d) : 0;
  // key tiles an item loads: [t0, te)
  auto item_t0 = [&](int c_) __attribute__((always_inline)) -> int { return SPLIT ? c_ * kc : 0; };
  auto item_te = [&](int qt_, int n_, int c_) __attribute__((always_inline)) -> int {
    const int nkv_ = (min(qt_ * kBMA + kBMA, n_) + kBN - 1) / kBN;
    return SPLIT ? min(c_ * kc + kc, nkv_) : nkv_;
  };
  // token row of the segment start of unit u_
  auto seg_row0 = [&](int u_) __attribute__((always_inline)) -> int64_t {
    const int sl = sd.bh.div(u_);
    return static_cast<int64_t>(u_ - sl * BH) * a.T + static_cast<int64_t>(a.s0 + sl) * a.N;
  };
  auto kv_tiles = [&](int qt_, int n_) __attribute__((always_inline)) -> int {
    return (min(qt_ * kBMA + kBMA, n_) + kBN - 1) / kBN;
  };

  int r = 0, u, qt, n, c;
  if (!find(r, u, qt, n, c)) return;

  // Q and K of the local attention (position-embedded when the caller supplies them)
  const uint16_t* qloc = static_cast<const uint16_t*>(a.q_loc);
  const uint16_t* kloc = static_cast<const uint16_t*>(a.k_loc);
  const uint16_t* vall = static_cast<const uint16_t*>(a.v);

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
  // K and V of tile i of the segment whose rows start at base (n_ tokens; rows at or past
  // the end arrive as zeros)
  auto issue_tile = [&](int64_t base, int n_, int i, uint16_t* dst) __attribute__((always_inline)) {
    const int kv0 = i * kBN;
    const uint32_t bytes = static_cast<uint32_t>(n_ - kv0) * D * 2;
    const uint16_t* ksrc = kloc + (base + kv0) * D;
    const uint16_t* vsrc = vall + (base + kv0) * D;
#pragma unroll
    for (int t = 0; t < CW; ++t) copy_group(wave * CW + t, ksrc, bytes, dst);
#pragma unroll
    for (int t = 0; t < CW; ++t) {
      const int c = wave * CW + t;
      copy1k(vsrc, bytes, 1024 * c, reinterpret_cast<char*>(dst + TILE) + 1024 * c, lp_v);
    }
  };
  // Q rows q0_ + 32 wave .. + 31 of the segment at base as the B operand of S^T: lane holds
  // Q[q][16 ks + 8 hl .. +7] (rows at or past n_ read as zeros)
  u32x4 qreg[KS];
  auto load_q = [&](const uint16_t* src, int64_t base, int n_, int qw0_) __attribute__((always_inline)) {
    const auto qr = buffer_rsrc(src + (base + qw0_) * D, static_cast<uint32_t>(max(n_ - qw0_, 0)) * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = buffer_ld16(qr, static_cast<uint32_t>(l32 * D + 16 * ks + 8 * hl) * 2);
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

  // ---- prologue of the first item: its Q rows straight into the B-operand registers,
  // tiles 0, 1 and 2 into buffers 0, 1 and 2.
  load_q(qloc, seg_row0(u), n, qt * kBMA + 32 * qb);
  {
    const int t0_ = item_t0(c), te_ = item_te(qt, n, c);
    issue_tile(seg_row0(u), n, t0_, buf0);
    if (t0_ + 1 < te_) issue_tile(seg_row0(u), n, t0_ + 1, buf1);
    if (t0_ + 2 < te_) issue_tile(seg_row0(u), n, t0_ + 2, buf2);
  }
  wait_vm_le(0);
  __builtin_amdgcn_s_barrier();

  const float c2 = a.scale_log2;
  constexpr int KH = KS / 2;   // k-steps per operand group
  typedef bf16x8 KOps[2][KH];  // [key half][k-step]

  // One item per pass.  On entry: the item's Q rows are in qreg (or in flight), its tiles
  // 0 .. 2 are in buffers 0 .. 2, complete and visible to every wave.
  for (;;) {
    const int h = sd.h.mod(sd.bh.mod(u));
    const int q0 = qt * kBMA;
    const int64_t row0 = seg_row0(u);
    const int nkv = kv_tiles(qt, n);
    const int jm = q0 / kBN;   // unmasked tiles (a multiple of 4); tiles jm .. jm + 3 hold the diagonal
    const int qw0 = q0 + 32 * qb;
    const int q = qw0 + l32;
    // The item's steps: unmasked tiles [t0, tu), then, if it holds the diagonal (the
    // query tile's last chunk), the four diagonal steps jm .. jm + 3; tend ends the step
    // sequence.  Every bound is a multiple of 4, so buffer j % 4 holds tile j throughout.
    const int t0 = item_t0(c), te = item_te(qt, n, c);
    const bool last = !SPLIT || te == nkv;
    const int tu = last ? jm : te;
    const int tend = last ? jm + 4 : tu;
    int rn = r + 1, un = 0, qtn = 0, nn = 0, cn = 0;
    const bool has_next = find(rn, un, qtn, nn, cn);
    const int64_t row0n = has_next ? seg_row0(un) : 0;
    const int t0n = has_next ? item_t0(cn) : 0;
    const int ten = has_next ? item_te(qtn, nn, cn) : 0;

    // Copy number i of the item's sequence: K and V of tile i for i < te; tiles t0n,
    // t0n + 1, t0n + 2 of the next item for i = tend .. tend + 2; nothing otherwise.
    // count: the copy instructions this wave issues for it.
    auto issue = [&](int i, uint16_t* dst) __attribute__((always_inline)) {
      if (i < te) issue_tile(row0, n, i, dst);
      else if (i >= tend && t0n + (i - tend) < ten) issue_tile(row0n, nn, t0n + (i - tend), dst);
    };
    auto count = [&](int i) __attribute__((always_inline)) -> int {
      return (i < te || (i >= tend && t0n + (i - tend) < ten)) ? 2 * CW : 0;
    };
    // M^T_{s-1} into its buffer: issued at the start of the item's second step, when every
    // wave is past the previous item's retrieval
    auto issue_mt = [&]() __attribute__((always_inline)) {
      const uint16_t* msrc = static_cast<const uint16_t*>(a.ws.mt) + static_cast<int64_t>(u) * D * D;
#pragma unroll
      // (a state still zero after a reset is read as zeros: an empty source range)
      for (int t = 0; t < MW; ++t) copy_group(wave * MW + t, msrc, a.zero_state ? 0u : D * D * 2u, bufm);
    };

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
      for (int i = 0; i < 16; ++i) sc[i] = (8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : sc[i];
    };
    auto half_max = [&](const f32x16& sc) __attribute__((always_inline)) -> float {
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      return mx;
    };
    // P = exp2(scale log2e S - m_run) in bf16 (the MFMA operand); the row sum adds the same
    // rounded values, so the output is normalised with exactly the weights it accumulated
    auto half_exp = [&](f32x16& sc, bf16x8& p_lo, bf16x8& p_hi) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -m_run));
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
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
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
    // Unmasked tiles j < jm run software-pipelined: iteration j holds the scores of tile j
    // (sc0 / sc1, maximum mxc) and computes those of tile j + 1 while it exponentiates and
    // multiplies tile j.  The exponentials are the largest VALU cost (a quarter-rate
    // instruction per score), so they are spread evenly over the iteration's MFMAs, in key
    // quarters (16 keys: 8 score registers of one half): quarter q of tile j is exponentiated
    // in group q and multiplied (O^T += V^T P^T, one MFMA per 32-row block of the head
    // dimension) in group q + 1, alternating with the score MFMAs of tile j + 1:
    //   group 0: S^T(j + 1) k-steps 0 .. KG - 1             | P quarter 0
    //   group 1: S^T(j + 1) next KG k-steps | PV quarter 0  | P quarter 1
    //   group 2: S^T(j + 1) next KG k-steps | PV quarter 1  | P quarter 2
    //   group 3: S^T(j + 1) last KG k-steps | PV quarter 2  | P quarter 3
    //   group 4:                              PV quarter 3  | maximum of tile j + 1
    // Every MFMA is a slot of its own (a scheduling barrier after it) holding its share of
    // the group's exponentials and of the LDS reads for the next group (the K^T operands of
    // its score k-steps, the V^T operands of its PV quarter), so no slot carries more VALU
    // work than the MFMA before it covers.  Products and row sums add in the same order as
    // with whole halves.  Buffer j % 4 holds tile j.  Copy j + 3 of the sequence is issued at
    // the start of iteration j into buffer (j + 3) % 4 (tile j - 1, done with at the previous
    // barrier) and waited for at its end, so tiles j + 1 and j + 2 are complete throughout
    // iteration j.
    constexpr int KG = KS / 4;    // score k-steps per group (2 KG = DB MFMAs of each kind)
    typedef bf16x8 KGrp[2][KG];   // [key half][k-step]
    typedef u32x2 VQ[DB][2];      // V^T operands of one key quarter, two transpose reads each
    auto read_k = [&](const uint16_t* kt, int k0, int r, KGrp& ak) __attribute__((always_inline)) {
      ak[r % 2][r / 2] = as_bf16x8(ld16(kt + g_rd + (r % 2) * 256 * CPR + 256 * (k0 + r / 2)));
    };
    auto read_v = [&](const uint16_t* kt, int q, int r, VQ& vq) __attribute__((always_inline)) {
      vq[r / 2][r % 2] = lds_read_tr16(kt + v_rd + 4 * q * 32 * CPR + 128 * (r / 2) + (r % 2) * 2 * 32 * CPR);
    };
    auto s_mfma = [&](const KGrp& ak, int k0, int m, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
      if (m % 2 == 0) s0 = mfma32x32x16(ak[0][m / 2], as_bf16x8(qreg[k0 + m / 2]), s0);
      else s1 = mfma32x32x16(ak[1][m / 2], as_bf16x8(qreg[k0 + m / 2]), s1);
    };
    auto pv_mfma = [&](const VQ& vq, int db, const u32x4& pq) __attribute__((always_inline)) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{vq[db][0][0], vq[db][0][1], vq[db][1][0], vq[db][1][1]});
      acc_o[db] = mfma32x32x16(av, as_bf16x8(pq), acc_o[db]);
    };
    // score e of a key quarter (registers r0 .. r0 + 7 of sc) -> P; an odd e also packs the
    // pair and adds it to the row sum
    auto p_elem = [&](f32x16& sc, int r0, int e, u32x4& pq) __attribute__((always_inline)) {
      sc[r0 + e] = __builtin_amdgcn_exp2f(fmaf(sc[r0 + e], c2, -m_run));
      if (e % 2 == 1) {
        pq[e / 2] = pack_bf16x2(sc[r0 + e - 1], sc[r0 + e]);
        l_part = add_bf16x2(pq[e / 2], l_part);
      }
    };
    f32x16 sc0, sc1;
    KOps kq;
    load_k(buf0, 0, kq);   // tile t0
    sc0 = zero16();
    sc1 = zero16();
    qk_part(kq, 0, sc0, sc1);
    load_k(buf0, KH, kq);
    qk_part(kq, KH, sc0, sc1);   // tile 0
    float mxc = tile_max(sc0, sc1);
    // Tile 2 (issued last in the previous item) is complete here in every wave, ahead of
    // its Q rows in the wave's load order; after the barrier it is visible to all.  (With
    // the free-running diagonal the previous item's last copies follow its Q rows: waited
    // for here.)
    if constexpr (kFree) wait_vm_le(0);
    __builtin_amdgcn_s_barrier();
    KGrp kg0;
    if (tu > t0) {   // tile t0 + 1, the first group's k-steps
      if constexpr (SPLIT) {
        load_k(buf1, 0, kq);
      } else {
#pragma unroll
        for (int r = 0; r < 2 * KG; ++r) read_k(buf1, 0, r, kg0);
      }
    }
    // The split-key kernel (one-segment calls) keeps the earlier schedule: per iteration,
    // S^T(j + 1) in two k-step halves with tile j's exponentials, then the two PV halves.
    // With its chunk bookkeeping live, the quarter schedule spills there and measured 6%
    // slower per segment.
    auto pstep_halves = [&](int j, auto bufc) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      maybe_rescale(mxc);
      if (j == t0 + 1) issue_mt();
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
    auto pstep = [&](int j, auto bufc) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      maybe_rescale(mxc);
      if (j == t0 + 1) issue_mt();
      issue(j + 3, bufp(IC<b + 3>{}));
      const uint16_t* kt = bufp(bufc);
      const uint16_t* kn = bufp(IC<b + 1>{});
      const uint16_t* kn2 = bufp(IC<b + 2>{});
      f32x16 n0 = zero16(), n1 = zero16();
      u32x4 pq[4];
      KGrp kg1;
      VQ va, vb;
      __builtin_amdgcn_sched_barrier(0);
      // group 0: DB score MFMAs; reads: K^T of group 1, V^T of quarter 0
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        s_mfma(kg0, 0, i, n0, n1);
#pragma unroll
        for (int r = 3 * DB * i / DB; r < 3 * DB * (i + 1) / DB; ++r) {
          if (r < DB) read_k(kn, KG, r, kg1);
          else read_v(kt, 0, r - DB, va);
        }
#pragma unroll
        for (int e = 8 * i / DB; e < 8 * (i + 1) / DB; ++e) p_elem(sc0, 0, e, pq[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // groups 1 .. 3: score and PV MFMAs alternating
      auto mid = [&](auto gc, const KGrp& ak, KGrp& an, const VQ& vu, VQ& vn, f32x16& sq) __attribute__((always_inline)) {
        constexpr int G = decltype(gc)::value;
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
          if (i % 2 == 0) s_mfma(ak, G * KG, i / 2, n0, n1);
          else pv_mfma(vu, i / 2, pq[G - 1]);
          // reads: K^T of group G + 1 (of tile j + 2's group 0 in group 3), V^T of quarter G
#pragma unroll
          for (int r = 3 * DB * i / (2 * DB); r < 3 * DB * (i + 1) / (2 * DB); ++r) {
            // group 4 runs PV only: group 3 reads its V^T first
            const int rk = G < 3 ? r : r - 2 * DB, rv = G < 3 ? r - DB : r;
            if (rk >= 0 && rk < DB) read_k(G < 3 ? kn : kn2, G < 3 ? (G + 1) * KG : 0, rk, an);
            else read_v(kt, G, rv, vn);
          }
#pragma unroll
          for (int e = 8 * i / (2 * DB); e < 8 * (i + 1) / (2 * DB); ++e) p_elem(sq, 8 * (G % 2), e, pq[G]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      mid(IC<1>{}, kg1, kg0, va, vb, sc0);
      mid(IC<2>{}, kg0, kg1, vb, va, sc1);
      mid(IC<3>{}, kg1, kg0, va, vb, sc1);   // kg0 <- tile j + 2, read but unused past the last tile
      // group 4: PV quarter 3, the maximum of tile j + 1
      float mh0 = 0.f, mh1 = 0.f;
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        pv_mfma(vb, i, pq[3]);
        if (i == 0) mh0 = half_max(n0);
        if (i == 1) mh1 = half_max(n1);
        if (i == DB - 1) mxc = max_across_halves(fmaxf(mh0, mh1)) * c2;
        __builtin_amdgcn_sched_barrier(0);
      }
      sc0 = n0;
      sc1 = n1;
      wait_vm_le(0);
      __builtin_amdgcn_s_barrier();
    };
    for (int j = t0; j < tu; j += 4) {
      if constexpr (SPLIT) {
        pstep_halves(j, IC<0>{});
        pstep_halves(j + 1, IC<1>{});
        pstep_halves(j + 2, IC<2>{});
        pstep_halves(j + 3, IC<3>{});
      } else {
        pstep(j, IC<0>{});
        pstep(j + 1, IC<1>{});
        pstep(j + 2, IC<2>{});
        pstep(j + 3, IC<3>{});
      }
    }
    // The four tiles from q0 on hold the diagonal of every wave: masked, one at a time;
    // tile jm's scores are already in sc0 / sc1.  A wave skips a tile whose keys all lie
    // past its queries, and every wave skips tiles past the segment end; the four steps
    // run in every item, since their copies feed the next item's tiles 0 .. 2.  Each step
    // waits for the copy the next step reads (the last one for all copies: the next
    // item's tiles and M^T_{s-1}).
    auto mstep = [&](int j, auto bufc, bool have_scores) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      const uint16_t* kt = bufp(bufc);
      if (j == t0 + 1) issue_mt();
      issue(j + 3, bufp(IC<b + 3>{}));
      const int kv0 = j * kBN;
      if (j < nkv && kv0 <= qw0 + 31) {
        if (!have_scores) qk_tile(kt, sc0, sc1);
        mask_half(sc0, kv0);
        mask_half(sc1, kv0 + 32);
        maybe_rescale(tile_max(sc0, sc1));
        finish_tile(kt, sc0, sc1);
      }
      if constexpr (b == 3) wait_vm_le(count(j + 3));
      else wait_vm_le(count(j + 2) + count(j + 3));
      __builtin_amdgcn_s_barrier();
    };
    if (last) {
      if constexpr (kFree) {
        // Tile jm serves every wave; the step waits for all copies (tiles jm + 1 .. jm + 3
        // complete), and after its barrier buffer 0 takes the next item's first tile.  Then
        // every wave runs its remaining diagonal tiles and its epilogue without barriers;
        // the item ends with one, after which buffers 1 and 2 take the next item's tiles.
        if (jm == t0) issue_mt();   // an item without unmasked tiles: M^T_{s-1} not yet copied
        issue(jm + 3, buf3);
        mask_half(sc0, jm * kBN);
        mask_half(sc1, jm * kBN + 32);
        maybe_rescale(tile_max(sc0, sc1));
        finish_tile(buf0, sc0, sc1);
        wait_vm_le(0);
        __builtin_amdgcn_s_barrier();
        issue(tend, buf0);
        auto dtile = [&](auto ic) __attribute__((always_inline)) {
          const int j = jm + decltype(ic)::value, kv0 = j * kBN;
          if (j < nkv && kv0 <= qw0 + 31) {
            qk_tile(bufp(ic), sc0, sc1);
            mask_half(sc0, kv0);
            mask_half(sc1, kv0 + 32);
            maybe_rescale(tile_max(sc0, sc1));
            finish_tile(bufp(ic), sc0, sc1);
          }
        };
        // the wave of each SIMD with the longer rest (blocks 4 .. 7: two or three more tiles,
        // against none or one) issues first until its item ends
        if (qb >= 4) __builtin_amdgcn_s_setprio(2);
        dtile(IC<1>{});
        dtile(IC<2>{});
        dtile(IC<3>{});
      } else {
        mstep(jm, IC<0>{}, true);
        mstep(jm + 1, IC<1>{}, false);
        mstep(jm + 2, IC<2>{}, false);
        mstep(jm + 3, IC<3>{}, false);
      }
    }
    // (A chunk without the diagonal has computed scores of the next item's first tile in
    // its last step: they are not used.)

    // ---------------------------------------------------------------- epilogue
    // M^T_{s-1} is in bufm.  The next item's first tiles are in buffers 0 .. 2 (with the
    // free-running diagonal only its first, in buffer 0: the other two are copied after the
    // item's closing barrier); this item's Q registers are free once sigma(Q) is formed, and
    // take the next item's Q.
    bool finish = true;
    if constexpr (SPLIT) {
      const int nchunks = sd.kc.div(nkv + kc - 1);
      if (nchunks > 1) {
        // Hand the partial softmax state (O^T unnormalised, in bf16; the running maximum
        // and row sum in fp32) to the query tile's slot c with device-coherent stores; once
        // every wave's stores have completed, count the chunk.  The workgroup that counts
        // the last chunk merges all of them in chunk order, using for its own chunk the same
        // bf16 values it stored (the same arithmetic whichever workgroup merges), and
        // finishes the tile; the others go on to their next item.  Nothing waits.
        const int tile = u * nq + qt;
        int base = 0;   // chunks of the query tiles before qt in a full segment
        for (int t = 0; t < qt; ++t) base += sd.kc.div((min(t * kBMA + kBMA, a.N) + kBN - 1) / kBN + kc - 1);
        const int64_t slot0 = static_cast<int64_t>(u) * a.split_slots + base;
        constexpr int PG = 2 * DB;                       // 16-byte groups per lane (8 values each)
        constexpr uint32_t kAccBytes = 8u * PG * 64u * 16u, kMlBytes = 512u * 8u;
        auto acc_rsrc = [&](int ch) __attribute__((always_inline)) {
          return buffer_rsrc(static_cast<const char*>(a.split_acc) + (slot0 + ch) * kAccBytes, kAccBytes);
        };
        auto ml_rsrc = [&](int ch) __attribute__((always_inline)) {
          return buffer_rsrc(a.split_ml + (slot0 + ch) * 1024, kMlBytes);
        };
        auto acc_off = [&](int g) __attribute__((always_inline)) -> uint32_t {
          return static_cast<uint32_t>(((wave * PG + g) * 64 + lane) * 16);
        };
        // group g = 2 db + hh holds acc_o[db][8 hh .. 8 hh + 7]
        u32x4 own[PG];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              own[2 * db + hh][e] = pack_bf16x2(acc_o[db][8 * hh + 2 * e], acc_o[db][8 * hh + 2 * e + 1]);
        {
          const auto ar = acc_rsrc(c);
#pragma unroll
          for (int g = 0; g < PG; ++g) buffer_st16_dev(ar, acc_off(g), own[g]);
          buffer_st8_dev(ml_rsrc(c), static_cast<uint32_t>((wave * 64 + lane) * 8),
                         u32x2{__float_as_uint(m_run), __float_as_uint(l_part)});
        }
        wait_vm_le(0);
        __builtin_amdgcn_s_barrier();
        // buffer 3 is free here (its last tile is consumed; the next item's copy into it
        // is issued after the next item's first barrier): it carries the count to all waves
        int* flag = reinterpret_cast<int*>(buf3);
        if (tid == 0)
          flag[0] = __hip_atomic_fetch_add(a.split_cnt + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int done = __builtin_amdgcn_readfirstlane(flag[0]);
        finish = done == nchunks - 1;
        if (!finish) {
          if (has_next) load_q(qloc, row0n, nn, qtn * kBMA + 32 * wave);
        } else {
          if (tid == 0) __hip_atomic_store(a.split_cnt + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          float mc[kMaxChunks], lc[kMaxChunks];
          float m_all = -INFINITY;
#pragma unroll
          for (int ch = 0; ch < kMaxChunks; ++ch) {
            if (ch < nchunks) {
              const u32x2 ml = buffer_ld8_dev(ml_rsrc(ch), static_cast<uint32_t>((wave * 64 + lane) * 8));
              mc[ch] = __uint_as_float(ml[0]);
              lc[ch] = __uint_as_float(ml[1]);
              m_all = fmaxf(m_all, mc[ch]);
            }
          }
          float lsum = 0.f;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc_o[db] = zero16();
          // chunks in windows of kWin: the other chunks' loads of a window are all in
          // flight before the window is added (in chunk order)
          constexpr int kWin = 2;
#pragma unroll
          for (int w0 = 0; w0 < kMaxChunks; w0 += kWin) {
            if (w0 < nchunks) {
              u32x4 pb[kWin][PG];
#pragma unroll
              for (int j = 0; j < kWin; ++j) {
                const int ch = w0 + j;
                if (ch < nchunks && ch != c) {
                  const auto ar = acc_rsrc(ch);
#pragma unroll
                  for (int g = 0; g < PG; ++g) pb[j][g] = buffer_ld16_dev(ar, acc_off(g));
                }
              }
#pragma unroll
              for (int j = 0; j < kWin; ++j) {
                const int ch = w0 + j;
                if (ch < nchunks) {
                  const float f = __builtin_amdgcn_exp2f(mc[ch] - m_all);
                  lsum = fmaf(f, lc[ch], lsum);
                  const bool mine = ch == c;
#pragma unroll
                  for (int g = 0; g < PG; ++g) {
                    const u32x4 v = mine ? own[g] : pb[j][g];
                    const int db = g / 2, o = 8 * (g % 2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                      acc_o[db][o + 2 * e] = fmaf(f, bf16lo_to_f32(v[e]), acc_o[db][o + 2 * e]);
                      acc_o[db][o + 2 * e + 1] = fmaf(f, bf16hi_to_f32(v[e]), acc_o[db][o + 2 * e + 1]);
                    }
                  }
                }
              }
            }
          }
          l_part = lsum;
          m_run = m_all;
        }
      }
    }
    if (finish) {
    const float l_tot = sum_across_halves(l_part);
    const float inv_l = 1.f / l_tot;
    if constexpr (MODE >= 1) {
      if (a.lse && hl == 0 && q < n) a.lse[row0 + q] = m_run + __log2f(l_tot);
    }
    // z_{s-1}: this lane's 8 entries of each k-step (two addresses per load: one per half)
    f32x4 zr[KS][2];
    {
      const f32x4* zq = reinterpret_cast<const f32x4*>(a.ws.zb + static_cast<int64_t>(u) * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        zr[ks][0] = a.zero_state ? f32x4{0.f, 0.f, 0.f, 0.f} : zq[4 * ks + 2 * hl];
        zr[ks][1] = a.zero_state ? f32x4{0.f, 0.f, 0.f, 0.f} : zq[4 * ks + 2 * hl + 1];
      }
    }
    // With a separate local Q the retrieval reads the PE-free Q rows.
    if (a.q_loc != a.q) load_q(static_cast<const uint16_t*>(a.q), row0, n, qw0);

    // sigma(Q) as the B operand of the retrieval, and the denominator sigma(q) . z_{s-1}
    float den = 0.f;
    bf16x8 sq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[2 * i] = elu_plus_one(bf16lo_to_f32(qreg[ks][i]));
        sv[2 * i + 1] = elu_plus_one(bf16hi_to_f32(qreg[ks][i]));
      }
      const f32x4 z0 = zr[ks][0], z1 = zr[ks][1];
      den += sv[0] * z0[0] + sv[1] * z0[1] + sv[2] * z0[2] + sv[3] * z0[3] +
             sv[4] * z1[0] + sv[5] * z1[1] + sv[6] * z1[2] + sv[7] * z1[3];
      sq[ks] = as_bf16x8(u32x4{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                               pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7])});
    }
    if (has_next) load_q(qloc, row0n, nn, qtn * kBMA + 32 * qb);
    den = sum_across_halves(den);
    const float inv_den = 1.f / (den + a.eps);
    const float g = a.gate_g[h], omg = a.gate_omg[h];
    float ddp = 0.f, emp = 0.f;   // MODE 2: this lane's shares of dO . A_dot and dO . A_mem
    const uint16_t* dog = MODE == 2 ? static_cast<const uint16_t*>(a.bwd_dout) + (row0 + q) * D : nullptr;
    // the output rows qw0 .. qw0 + 31 (stores to rows at or past n are dropped)
    const auto orsrc = buffer_rsrc(static_cast<uint16_t*>(a.out) + (row0 + qw0) * D,
                                   static_cast<uint32_t>(max(n - qw0, 0)) * D * 2);

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16 acc_m = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 am = as_bf16x8(ld16(bufm + g_rd + db * 256 * CPR + 256 * ks));
        acc_m = mfma32x32x16(am, sq[ks], acc_m);
      }
      float o[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float amem = acc_m[i] * inv_den;
        const float adot = acc_o[db][i] * inv_l;
        o[i] = g * amem + omg * adot;
        if constexpr (MODE == 1) {
          if (q < n) {
            const int dv = 32 * db + 8 * (i >> 2) + 4 * hl + (i & 3);
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
        // Lane (l, hl) holds columns 32 db + 8 r4 + 4 hl .. +3 of row q for r4 = 0 .. 3.
        // One swap of lane halves per dword pairs them into whole 16-byte chunks: the
        // low half then holds chunks 1 and 3 of the 32 columns, the high half chunks 0
        // and 2, each as (columns 0..3 from one lane, 4..7 from the other).
        uint32_t pk[4][2];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          pk[r4][0] = pack_bf16x2(o[4 * r4], o[4 * r4 + 1]);
          pk[r4][1] = pack_bf16x2(o[4 * r4 + 2], o[4 * r4 + 3]);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * pr + 1][0], pk[2 * pr][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * pr + 1][1], pk[2 * pr][1], false, false);
          const int chunk = 4 * db + 2 * pr + (hl ? 0 : 1);
          buffer_st16(orsrc, static_cast<uint32_t>(l32 * D + 8 * chunk) * 2, u32x4{s0[0], s1[0], s0[1], s1[1]});
        }
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
    }
    }   // finish
    if constexpr (kFree) {
      __builtin_amdgcn_s_setprio(0);
      // every wave's copy into buffer 0 is complete (in the plain output mode only the next
      // Q rows and the output stores may follow it); after the barrier no wave reads
      // buffers 1 .. 3 or M^T
      wait_vm_le(MODE == 0 ? KS + 2 * DB : 0);
      __builtin_amdgcn_s_barrier();
      issue(tend + 1, buf1);
      issue(tend + 2, buf2);
    }
    if (!has_next) break;
    r = rn;
    u = un;
    qt = qtn;
    n = nn;
    c = cn;
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

// Compute units of the current device (the persistent grid's size), looked up once per device.
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <int D>
hipError_t launch_attention_d(const WindowArgs& a, hipStream_t st) {
  if (a.bf16) {
    const int units = a.units(), nq = (a.N + kBMA - 1) / kBMA;
    const dim3 grid(min(units * nq, compute_units()));
    Sched sd;
    sd.units = FastDiv(static_cast<uint32_t>(units));
    sd.grp = FastDiv(static_cast<uint32_t>(kGroup * nq));
    sd.last = FastDiv(static_cast<uint32_t>((units / 8) % kGroup));
    sd.bh = FastDiv(static_cast<uint32_t>(a.B * a.H));
    sd.h = FastDiv(static_cast<uint32_t>(a.H));
    if (a.split_kc > 0) {
      // split-key mode: one segment, MODE 0, items counted by the host
      if (a.W != 1 || a.bwd_dout || a.a_mem || a.a_dot || a.lse || a.split_kc % 4 != 0 ||
          a.split_kc * kMaxChunks < 4 * nq || a.split_items < 1 ||
          a.split_slots < a.split_items || !a.split_acc || !a.split_ml || !a.split_cnt)
        return hipErrorInvalidValue;
      sd.kc = FastDiv(static_cast<uint32_t>(a.split_kc));
      sd.items = a.split_items;
      const dim3 sgrid(min(units * a.split_items, compute_units()));
      hipLaunchKernelGGL((k_attn_bf16<D, 0, true>), sgrid, dim3(kThreadsA), 0, st, a, sd);
    } else if (a.bwd_dout) {
      hipLaunchKernelGGL((k_attn_bf16<D, 2, false>), grid, dim3(kThreadsA), 0, st, a, sd);
    } else if (a.a_mem || a.a_dot || a.lse) {
      hipLaunchKernelGGL((k_attn_bf16<D, 1, false>), grid, dim3(kThreadsA), 0, st, a, sd);
    } else {
      hipLaunchKernelGGL((k_attn_bf16<D, 0, false>), grid, dim3(kThreadsA), 0, st, a, sd);
    }
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
