// Matrix-core kernels of the backward pass's local-attention gradients (Eq. 6, bf16 path),
// plus the retrieval part of dQ (Eq. 7).  See backward.hip for the formulas; here
// P = exp2(c q.k - lse) is recomputed from the forward's log-sum-exp, D_t = dO_t . A_dot_t and
// the upstream gradient dO is used unscaled (the (1 - g) factor of the local arm is applied
// to the results).
//
// dQ (k_bwd_dq_mfma): one workgroup = 4 waves = 128 queries of one (segment, batch, head);
// every wave owns 32 queries and works in the forward kernel's transposed frame:
//   S^T = K Q^T and dP^T = V dO^T (Q and dO rows are the B operands, held in registers),
//   dS^T = P^T o (dP^T - D), dQ^T += K^T dS^T (the dS^T registers, converted to bf16, are the
//   B operand, with K^T read from LDS by transpose reads in the key order they hold),
// so softmax statistics are per-lane scalars.  K and V tiles of 64 keys go HBM -> LDS by
// buffer -> LDS copies, double buffered.  The epilogue adds the retrieval part
// (g / den) M dO^T + dden z, with M_{s-1} read from the forward's M^T copy by transpose
// reads, multiplies by sigma'(Q), and stores fp32 dQ rows.
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kBwdThreads = 256;   // 4 waves
constexpr int kBwdQ = 128;         // queries per workgroup
constexpr int kBwdK = 64;          // keys per tile

// Copy `rows` rows of a [*, D] bf16 array into LDS in the 16-row-group layout (chunk c of
// row r in slot (r / 16) * 16 CPR + 16 c + r % 16): copy number c of the tile (1 KB) covers
// rows 16 g + lane % 16, chunks 4 j + lane / 16 with g = c / (CPR / 4), j = c % (CPR / 4).
// Rows at or past `valid_rows` read as zeros.  The caller spreads the copies over its waves.
template <int D>
__device__ __forceinline__ void copy_rows(const uint16_t* src, int valid_rows, uint16_t* lds, int c, int lane) {
  constexpr int CPR = D / 8;
  const int g = c / (CPR / 4), j = c % (CPR / 4);
  const int shift = g * 32 * D + 64 * j;   // bytes
  const int left = __builtin_amdgcn_readfirstlane(max(valid_rows * 2 * D - shift, 0));
  const uint32_t lp = static_cast<uint32_t>((lane & 15) * 2 * D + 16 * (lane >> 4));
  copy_to_lds(reinterpret_cast<const char*>(src) + shift, static_cast<uint32_t>(left), lds + 512 * c, lp);
}

template <int D>
__global__ __launch_bounds__(kBwdThreads, 2) void k_bwd_dq_mfma(const BackwardArgs b) {
  constexpr int KS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int TILE = kBwdK * D;           // elements of a K (or V) tile
  constexpr int CPT = kBwdK * D * 2 / 1024; // 1 KB copies per tensor tile
  constexpr int CPW = CPT / 4;              // ... per wave
  static_assert(D * D <= 2 * TILE, "M^T fits one buffer");
  __shared__ __align__(16) uint16_t buf0[2 * TILE];
  __shared__ __align__(16) uint16_t buf1[2 * TILE];

  const WindowArgs& w = b.w;
  const int units = w.units();
  const int nq = (w.N + kBwdQ - 1) / kBwdQ;
  const int u = static_cast<int>(blockIdx.x) % units;
  const int qt = nq - 1 - static_cast<int>(blockIdx.x) / units;   // longest tiles first
  const int BH = w.B * w.H;
  const int s_local = u / BH, bh = u % BH, h = bh % w.H;
  const int n = w.seg_tokens(s_local);
  const int q0 = qt * kBwdQ;
  if (q0 >= n) return;
  const int64_t row0 = static_cast<int64_t>(bh) * w.T + static_cast<int64_t>(w.s0 + s_local) * w.N;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + l32;
  const bool live = q < n;
  const int64_t row = row0 + q;

  const uint16_t* qg = static_cast<const uint16_t*>(w.q_loc) + row0 * D;
  const uint16_t* kg = static_cast<const uint16_t*>(w.k_loc) + row0 * D;
  const uint16_t* vg = static_cast<const uint16_t*>(w.v) + row0 * D;
  const uint16_t* og = static_cast<const uint16_t*>(b.dout) + row0 * D;

  // this lane's query as the B operand: Q[q][16 ks + 8 hl .. +7], dO likewise
  u32x4 qreg[KS], oreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qreg[ks] = live ? ld16(qg + static_cast<int64_t>(q) * D + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
    oreg[ks] = live ? ld16(og + static_cast<int64_t>(q) * D + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  }
  const float lse = live ? w.lse[row] : INFINITY;   // P = 0 for rows past the segment
  const float dd = live ? b.dd[row] : 0.f;
  const float c2 = w.scale_log2;

  const int kv_end = min(q0 + kBwdQ, n);
  const int nkv = (kv_end + kBwdK - 1) / kBwdK;
  // tile i (keys 64 i ..) into dst: CPW copies of K and of V per wave; past the last tile
  // the copies are zero fills, so every tile is 2 CPW copies and the waits are constants
  auto issue = [&](int i, uint16_t* dst) __attribute__((always_inline)) {
    const int rows = i < nkv ? n - i * kBwdK : 0;
    const int64_t off = static_cast<int64_t>(min(i, nkv) * kBwdK) * D;
#pragma unroll
    for (int t = 0; t < CPW; ++t) copy_rows<D>(kg + off, rows, dst, wave * CPW + t, lane);
#pragma unroll
    for (int t = 0; t < CPW; ++t) copy_rows<D>(vg + off, rows, dst + TILE, wave * CPW + t, lane);
  };

  // LDS read offsets (elements)
  //  row-group operand read (K, V rows as the A operand): row 32 blk + l32, chunk 2 ks + hl
  const int g_rd = ((l32 >> 4) * 16 * CPR + 16 * hl + (l32 & 15)) * 8;
  //  K^T by transpose reads: lane j of 16-lane group G addresses key row
  //  16 j4 + 4 (G / 2) + j / 4 (+ 8), columns 32 db + 16 (G % 2) + 4 (j % 4) .. +3
  const int G = lane >> 4, jl = lane & 15;
  const int t_rd = (16 * (2 * (G & 1) + ((jl & 3) >> 1)) + 4 * (G >> 1) + (jl >> 2)) * 8 + 4 * (jl & 1);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();

  auto compute = [&](const uint16_t* kt, int j) __attribute__((always_inline)) {
    const int kv0 = j * kBwdK;
    if (kv0 > qw0 + 31) return;   // every key of the tile lies past this wave's queries
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
      dp[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[kb] = mfma32x32x16(as_bf16x8(ld16(kt + g_rd + kb * 256 * CPR + 256 * ks)), as_bf16x8(qreg[ks]), s[kb]);
        dp[kb] = mfma32x32x16(as_bf16x8(ld16(kt + TILE + g_rd + kb * 256 * CPR + 256 * ks)), as_bf16x8(oreg[ks]),
                              dp[kb]);
      }
    }
    // register r of block kb holds key kv0 + 32 kb + 8 (r / 4) + 4 hl + r % 4
    const bool masked = kv0 + kBwdK - 1 > qw0 || kv0 + kBwdK > n;
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -lse));
        if (masked) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          pr = (key > q || key >= n) ? 0.f : pr;
        }
        v[r] = pr * (dp[kb][r] - dd);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        dsb[2 * kb + half] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(v[8 * half], v[8 * half + 1]), pack_bf16x2(v[8 * half + 2], v[8 * half + 3]),
                          pack_bf16x2(v[8 * half + 4], v[8 * half + 5]), pack_bf16x2(v[8 * half + 6], v[8 * half + 7])});
    }
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* p = kt + t_rd + j4 * 128 * CPR + db * 512;
        const u32x2 a0 = lds_read_tr16(p);
        const u32x2 a1 = lds_read_tr16(p + 64);
        acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]}), dsb[j4], acc[db]);
      }
  };

  issue(0, buf0);
  issue(1, buf1);
  for (int j = 0; j < nkv; j += 2) {
    wait_vm_lgkm0<2 * CPW>();   // tile j (tile j + 1 may still be in flight)
    __builtin_amdgcn_s_barrier();
    compute(buf0, j);
    wait_vm_lgkm0<2 * CPW>();   // this wave's reads of buffer 0 are done
    __builtin_amdgcn_s_barrier();
    issue(j + 2, buf0);
    if (j + 1 < nkv) {
      wait_vm_lgkm0<2 * CPW>();   // tile j + 1
      __builtin_amdgcn_s_barrier();
      compute(buf1, j + 1);
      wait_vm_lgkm0<2 * CPW>();
      __builtin_amdgcn_s_barrier();
      issue(j + 3, buf1);
    }
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();

  // ---- retrieval part: X^T = M dO^T (rows i, columns queries), M_{s-1}[i][j] = mt[j][i]
  // The epilogue's own operands are loaded first, with no per-lane branch (rows past the
  // segment end read zeros and their stores are dropped), so that their latency overlaps the
  // copies of M^T: the PE-free Q values of this lane's query in result-register order,
  // z_{s-1} (staged in LDS), and the per-query den, dden.
  const uint32_t seg_el = static_cast<uint32_t>(n) * D;
  const auto qrs = buffer_rsrc(static_cast<const uint16_t*>(w.q) + row0 * D, seg_el * 2);
  const auto dqrs = buffer_rsrc(b.dq + row0 * D, seg_el * 4);
  const uint32_t e0 = static_cast<uint32_t>(q) * D;
  u32x2 qv[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) qv[db][r4] = buffer_ld8(qrs, 2 * (e0 + 32 * db + 8 * r4 + 4 * hl));
  const int64_t srow = live ? row : row0;   // a valid row for lanes past the end
  const float den_ld = b.den[srow], dden_ld = b.dden[srow];
  const float z_mine = threadIdx.x < D ? w.ws.zb[static_cast<int64_t>(u) * D + threadIdx.x] : 0.f;
  const uint16_t* mt = static_cast<const uint16_t*>(w.ws.mt) + static_cast<int64_t>(u) * D * D;
#pragma unroll
  for (int t = 0; t < D * D * 2 / 1024 / 4; ++t) copy_rows<D>(mt, D, buf0, wave * (D * D * 2 / 1024 / 4) + t, lane);
  float* zsh = reinterpret_cast<float*>(buf1);   // buffer 1 is free: its last tile was read
  if (threadIdx.x < D) zsh[threadIdx.x] = z_mine;
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  //  A operand M[i][16 ks + 8 hl + 0..7] = mt rows 16 ks + 8 hl + 0..7 at column i: lane j of
  //  group G addresses mt row 16 ks + 8 (G / 2) + j / 4 (+ 4), columns 32 db + 16 (G % 2) + 4 (j % 4)
  const int m_rd = (16 * (2 * (G & 1) + ((jl & 3) >> 1)) + 8 * (G >> 1) + (jl >> 2)) * 8 + 4 * (jl & 1);
  const float g = w.gate_g[h], omg = w.gate_omg[h];
  const float den = live ? den_ld : 1.f, dden = live ? dden_ld : 0.f;
  const float gd = g / den;
  const float sc = w.scale * omg;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 x = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint16_t* p = buf0 + m_rd + ks * 128 * CPR + db * 512;
      const u32x2 a0 = lds_read_tr16(p);
      const u32x2 a1 = lds_read_tr16(p + 32);
      x = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]}), as_bf16x8(oreg[ks]), x);
    }
    // register quad r4 holds features 32 db + 8 r4 + 4 hl + 0..3 of this lane's query
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int i0 = 32 * db + 8 * r4 + 4 * hl;
      const f32x4 zv = *reinterpret_cast<const f32x4*>(zsh + i0);
      const u32x2 qq = qv[db][r4];
      const float qf[4] = {bf16lo_to_f32(qq[0]), bf16hi_to_f32(qq[0]), bf16lo_to_f32(qq[1]), bf16hi_to_f32(qq[1])};
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qe = qf[e];
        const float ds = qe > 0.f ? 1.f : __builtin_amdgcn_exp2f(qe * kLog2e);
        o[e] = __float_as_uint(acc[db][4 * r4 + e] * sc + (gd * x[4 * r4 + e] + dden * zv[e]) * ds);
      }
      buffer_st16(dqrs, 4 * (e0 + i0), o);
    }
  }
}

// Element (r, c) of a [D][D] bf16 matrix in the 16-row-group layout: chunk c / 8 of row r
// in slot (r / 16) * 16 CPR + 16 (c / 8) + r % 16 (CPR = D / 8 chunks of 8 per row), so the 32
// rows of an MFMA A operand read 16-byte chunks at consecutive addresses.
__device__ __forceinline__ int rg_index(int r, int c, int cpr) {
  return ((r >> 4) * 16 * cpr + 16 * (c >> 3) + (r & 15)) * 8 + (c & 7);
}

// G_s (fp32, row-major [i][j]) -> bf16 in the 16-row-group layout in both orientations:
// gr holds rows i (G_s), gt rows j (G_s^T).  gr / gt may be LDS or global memory; the
// `threads` threads of the caller split the D * D / 8 chunks.
template <int D>
__device__ __forceinline__ void pack_g(const float* gm, uint16_t* gr, uint16_t* gt, int tid, int threads) {
  constexpr int CPR = D / 8;
#pragma unroll 4
  for (int e = tid; e < D * CPR; e += threads) {
    {  // G rows: chunk (i, cj)
      const int i = e / CPR, cj = e % CPR;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(gm + i * D + 8 * cj);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(gm + i * D + 8 * cj + 4);
      st16(gr + rg_index(i, 8 * cj, CPR), u32x4{pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                                               pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3])});
    }
    {  // G^T rows: chunk (j, ci) = G[8 ci .. + 7][j]
      const int j = e % D, ci = e / D;
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = gm[(8 * ci + k) * D + j];
      st16(gt + rg_index(j, 8 * ci, CPR), u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])});
    }
  }
}

// Packed G_s of every segment for the linear rule's fused dK, dV epilogue (one workgroup per
// segment and head).
template <int D>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_gpack(const BackwardArgs b) {
  const int64_t u = blockIdx.x;
  uint16_t* dst = b.gpk + u * 2 * D * D;
  pack_g<D>(b.gm + u * D * D, dst, dst + D * D, static_cast<int>(threadIdx.x), kBwdThreads);
}

// dK, dV (k_bwd_dkv_mfma): one workgroup = 4 waves = 128 keys; every wave owns 32 keys and
// works in the mirror frame, keys on lanes: S = Q K^T and dP = dO V^T (this wave's K and V
// rows are the B operands, held in registers), P and dS = P o (dP - D) per query row, then
// dV^T += dO^T P and dK^T += Q^T dS with the P / dS registers as B operands and dO^T, Q^T
// read from LDS by transpose reads in the query order those registers hold.  Query tiles of
// 64 (Q, dO, lse, D) go HBM -> LDS by buffer -> LDS copies, double buffered.
// (d = 128: the K, V operands and the dK, dV accumulators need more than 256 registers, so
// one workgroup per CU with the accumulators in AGPRs.)
// FUSE (linear rule): the memory-update part of dK, dV is added in the epilogue, in the
// accumulators' frame, before the one store: dV += sigma(K) G_s and
// dK += (V G_s^T + g_s) o sigma'(K) (Eq. 8 differentiated; G_s = dL/dM_s, g_s = dL/dz_s,
// both known: the reverse chains run before this kernel).  G_s arrives packed in bf16
// (k_bwd_gpack) and is copied to LDS while the query tiles stream.  Requires k_loc == k.
template <int D, bool FUSE>
__global__ __launch_bounds__(kBwdThreads, D == 128 ? 1 : 2) void k_bwd_dkv_mfma(const BackwardArgs b) {
  constexpr int KS = D / 16, DB = D / 32, CPR = D / 8, DD = D * D;
  constexpr int TILE = kBwdK * D;            // elements of a Q (or dO) tile
  constexpr int CPT = kBwdK * D * 2 / 1024;  // 1 KB copies per tensor tile
  constexpr int CPW = CPT / 4;
  constexpr int GCW = FUSE ? 2 * DD * 2 / 1024 / 4 : 0;   // 1 KB copies of packed G_s per wave
  __shared__ __align__(16) uint16_t buf0[2 * TILE];
  __shared__ __align__(16) uint16_t buf1[2 * TILE];
  __shared__ __align__(16) float st0[2][256];   // lse, D of the tile in buffer 0 (first 64 used)
  __shared__ __align__(16) float st1[2][256];
  __shared__ __align__(16) uint16_t gl[FUSE ? 2 * DD : 8];   // G_s rows i, then rows j
  __shared__ __align__(16) float gz_l[FUSE ? D : 4];          // g_s = dL/dz_s

  const WindowArgs& w = b.w;
  const int units = w.units();
  const int u = static_cast<int>(blockIdx.x) % units;
  const int kt = static_cast<int>(blockIdx.x) / units;   // key tile; the first ones are the longest
  const int BH = w.B * w.H;
  const int s_local = u / BH, bh = u % BH, h = bh % w.H;
  const int n = w.seg_tokens(s_local);
  const int k0 = kt * kBwdQ;
  if (k0 >= n) return;
  const int64_t row0 = static_cast<int64_t>(bh) * w.T + static_cast<int64_t>(w.s0 + s_local) * w.N;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;
  const bool live = key < n;
  // (FUSE) g_s, loaded now and staged in LDS for the epilogue
  const float gz_mine = FUSE && threadIdx.x < D ? b.gz[static_cast<int64_t>(u) * D + threadIdx.x] : 0.f;

  const uint16_t* qg = static_cast<const uint16_t*>(w.q_loc) + row0 * D;
  const uint16_t* kg = static_cast<const uint16_t*>(w.k_loc) + row0 * D;
  const uint16_t* vg = static_cast<const uint16_t*>(w.v) + row0 * D;
  const uint16_t* og = static_cast<const uint16_t*>(b.dout) + row0 * D;
  const float* lg = w.lse + row0;
  const float* dg = b.dd + row0;

  u32x4 kreg[KS], vreg[KS];   // this lane's key as the B operand
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kreg[ks] = live ? ld16(kg + static_cast<int64_t>(key) * D + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
    vreg[ks] = live ? ld16(vg + static_cast<int64_t>(key) * D + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  }
  const float c2 = w.scale_log2;

  const int t_first = k0 / kBwdK;                  // first query tile (queries >= the first key)
  const int nqt = (n + kBwdK - 1) / kBwdK - t_first;   // query tiles to visit
  // query tile t_first + i into (dst, stats): CPW copies of Q and of dO per wave, plus the
  // tile's lse (wave 0) and D (wave 1); past the last tile the copies are zero fills
  auto issue = [&](int i, uint16_t* dst, float (*stats)[256]) __attribute__((always_inline)) {
    const int t = t_first + min(i, nqt);
    const int rows = i < nqt ? n - t * kBwdK : 0;
    const int64_t off = static_cast<int64_t>(t * kBwdK) * D;
#pragma unroll
    for (int c = 0; c < CPW; ++c) copy_rows<D>(qg + off, rows, dst, wave * CPW + c, lane);
#pragma unroll
    for (int c = 0; c < CPW; ++c) copy_rows<D>(og + off, rows, dst + TILE, wave * CPW + c, lane);
    if (wave < 2) {   // 64 floats (lanes 16 .. 63 write zeros into the rest of the 1 KB row)
      const float* src = (wave == 0 ? lg : dg) + t * kBwdK;
      const uint32_t bytes = static_cast<uint32_t>(max(min(rows, kBwdK), 0)) * 4;
      copy_to_lds(src, bytes, reinterpret_cast<const uint16_t*>(stats[wave]), static_cast<uint32_t>(lane) * 16);
    }
  };

  const int g_rd = ((l32 >> 4) * 16 * CPR + 16 * hl + (l32 & 15)) * 8;
  const int G = lane >> 4, jl = lane & 15;
  const int t_rd = (16 * (2 * (G & 1) + ((jl & 3) >> 1)) + 4 * (G >> 1) + (jl >> 2)) * 8 + 4 * (jl & 1);

  f32x16 adv[DB], adk[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    adv[db] = zero16();
    adk[db] = zero16();
  }

  auto compute = [&](const uint16_t* qt_, const float (*stats)[256], int i) __attribute__((always_inline)) {
    const int t0 = (t_first + i) * kBwdK;
    if (t0 + kBwdK - 1 < kw0) return;   // every query of the tile precedes this wave's keys
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = zero16();
      dp[qb] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[qb] = mfma32x32x16(as_bf16x8(ld16(qt_ + g_rd + qb * 256 * CPR + 256 * ks)), as_bf16x8(kreg[ks]), s[qb]);
        dp[qb] = mfma32x32x16(as_bf16x8(ld16(qt_ + TILE + g_rd + qb * 256 * CPR + 256 * ks)), as_bf16x8(vreg[ks]),
                              dp[qb]);
      }
    }
    // register r of block qb holds query t0 + 32 qb + 8 (r / 4) + 4 hl + r % 4
    const bool masked = t0 < kw0 + 31 || t0 + kBwdK > n;
    bf16x8 pb[4], dsb[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[16], dv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rl = 32 * qb + 8 * r4 + 4 * hl;   // tile row of register 4 r4
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&stats[0][rl]);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&stats[1][rl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c2, -lv[e]));
          if (masked) {
            const int qr = t0 + rl + e;
            pr = (qr < key || qr >= n) ? 0.f : pr;
          }
          pv[r] = pr;
          dv[r] = pr * (dp[qb][r] - dv4[e]);
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        pb[2 * qb + half] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(pv[8 * half], pv[8 * half + 1]), pack_bf16x2(pv[8 * half + 2], pv[8 * half + 3]),
                          pack_bf16x2(pv[8 * half + 4], pv[8 * half + 5]),
                          pack_bf16x2(pv[8 * half + 6], pv[8 * half + 7])});
        dsb[2 * qb + half] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(dv[8 * half], dv[8 * half + 1]), pack_bf16x2(dv[8 * half + 2], dv[8 * half + 3]),
                          pack_bf16x2(dv[8 * half + 4], dv[8 * half + 5]),
                          pack_bf16x2(dv[8 * half + 6], dv[8 * half + 7])});
      }
    }
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* po = qt_ + TILE + t_rd + j4 * 128 * CPR + db * 512;
        const u32x2 o0 = lds_read_tr16(po);
        const u32x2 o1 = lds_read_tr16(po + 64);
        adv[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{o0[0], o0[1], o1[0], o1[1]}), pb[j4], adv[db]);
        const uint16_t* pq = qt_ + t_rd + j4 * 128 * CPR + db * 512;
        const u32x2 q0_ = lds_read_tr16(pq);
        const u32x2 q1_ = lds_read_tr16(pq + 64);
        adk[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{q0_[0], q0_[1], q1_[0], q1_[1]}), dsb[j4], adk[db]);
      }
  };

  issue(0, buf0, st0);
  issue(1, buf1, st1);
  if constexpr (FUSE) {   // after tiles 0 and 1: the first pass of the loop lets these be in flight
    const uint16_t* gsrc = b.gpk + static_cast<int64_t>(u) * 2 * DD;
#pragma unroll
    for (int c = 0; c < GCW; ++c) {
      const int idx = wave * GCW + c;
      copy_to_lds(gsrc + 512 * idx, 1024u, gl + 512 * idx, static_cast<uint32_t>(lane) * 16);
    }
  }
  // vmcnt of the tile waits, as immediates: the copies younger than the tile waited for are
  // this wave's copies of one tile, plus those of G_s during the first pair of tiles
  auto wait_tiles = [&](bool first) __attribute__((always_inline)) {
    constexpr int C = 2 * CPW;
    if (wave < 2) {
      if (first) wait_vm_lgkm0<C + 1 + GCW>();
      else wait_vm_lgkm0<C + 1>();
    } else {
      if (first) wait_vm_lgkm0<C + GCW>();
      else wait_vm_lgkm0<C>();
    }
  };
  for (int i = 0; i < nqt; i += 2) {
    const bool first = i == 0;
    wait_tiles(first);   // tile i (tile i + 1 may still be in flight)
    __builtin_amdgcn_s_barrier();
    compute(buf0, st0, i);
    wait_tiles(first);   // this wave's LDS reads of buffer 0 are done
    __builtin_amdgcn_s_barrier();
    issue(i + 2, buf0, st0);
    if (i + 1 < nqt) {
      wait_tiles(first);
      __builtin_amdgcn_s_barrier();
      compute(buf1, st1, i + 1);
      wait_tiles(first);
      __builtin_amdgcn_s_barrier();
      issue(i + 3, buf1, st1);
    }
  }
  wait_vm_le(0);   // no copy may land in LDS after the workgroup ends
  const float omg = w.gate_omg[h], sc = w.scale * omg;
  if constexpr (FUSE) {
    if (threadIdx.x < D) gz_l[threadIdx.x] = gz_mine;
    __syncthreads();   // every wave's copies of G_s have landed, g_s is staged
    const uint16_t* gr_l = gl;        // G_s, rows i
    const uint16_t* gt_l = gl + DD;   // G_s^T, rows j
    // sigma(k) of this lane's key as the B operand (zero past the segment's end)
    bf16x8 wreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float wf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = elu_plus_one(bf16lo_to_f32(kreg[ks][e])), hi = elu_plus_one(bf16hi_to_f32(kreg[ks][e]));
        wf[2 * e] = live ? lo : 0.f;
        wf[2 * e + 1] = live ? hi : 0.f;
      }
      wreg[ks] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(wf[0], wf[1]), pack_bf16x2(wf[2], wf[3]),
                                                 pack_bf16x2(wf[4], wf[5]), pack_bf16x2(wf[6], wf[7])});
    }
    // rows of dK, dV end at the segment's last key: stores of lanes past it are dropped
    const uint32_t nb = static_cast<uint32_t>(n) * D;
    const auto dvrs = buffer_rsrc(b.dv + row0 * D, nb * 4);
    const auto dkrs = buffer_rsrc(b.dk + row0 * D, nb * 4);
    const uint32_t e0 = static_cast<uint32_t>(key) * D;
    // dV^T = (1 - g) (local) + G_s^T sigma(K)^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) adv[db][r] *= omg;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        adv[db] = mfma32x32x16(as_bf16x8(ld16(gt_l + g_rd + db * 256 * CPR + 256 * ks)), wreg[ks], adv[db]);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        buffer_st16(dvrs, 4 * (e0 + 32 * db + 8 * r4 + 4 * hl),
                    u32x4{__float_as_uint(adv[db][4 * r4]), __float_as_uint(adv[db][4 * r4 + 1]),
                          __float_as_uint(adv[db][4 * r4 + 2]), __float_as_uint(adv[db][4 * r4 + 3])});
    }
    // dK^T = (1 - g) scale (local) + (G_s V^T + g_s) o sigma'(K)^T.  Register 4 q + e of block
    // ib is feature 32 ib + 8 q + 4 hl + e; kreg[ks] holds features 16 ks + 8 hl .. + 7, so
    // the key values of a block come from this lane and its partner lane ^ 32.
#pragma unroll
    for (int ib = 0; ib < DB; ++ib) {
      f32x16 sg = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sg = mfma32x32x16(as_bf16x8(ld16(gr_l + g_rd + ib * 256 * CPR + 256 * ks)), as_bf16x8(vreg[ks]), sg);
      u32x4 kh[2][2];   // [x][half]: kreg[2 ib + x] as held by the lane with hl = half
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t own = kreg[2 * ib + x][d];
          const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(own), 32));
          kh[x][0][d] = hl ? other : own;
          kh[x][1][d] = hl ? own : other;
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i0 = 32 * ib + 8 * q + 4 * hl;
        const f32x4 gz4 = *reinterpret_cast<const f32x4*>(&gz_l[i0]);
        const u32x4 src = kh[q >> 1][q & 1];   // features 32 ib + 16 (q >> 1) + 8 (q & 1) .. + 7
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t dw = hl ? src[2 + (e >> 1)] : src[e >> 1];
          const float kf = (e & 1) ? bf16hi_to_f32(dw) : bf16lo_to_f32(dw);
          const float dsig = kf > 0.f ? 1.f : __builtin_amdgcn_exp2f(kf * kLog2e);
          o[e] = __float_as_uint(fmaf(adk[ib][4 * q + e], sc, (sg[4 * q + e] + gz4[e]) * dsig));
        }
        buffer_st16(dkrs, 4 * (e0 + i0), o);
      }
    }
    return;
  }
  if (!live) return;
  const int64_t krow = row0 + key;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int i0 = 32 * db + 8 * r4 + 4 * hl;
      f32x4 ov, ok;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = adv[db][4 * r4 + e] * omg;
        ok[e] = adk[db][4 * r4 + e] * sc;
      }
      *reinterpret_cast<f32x4*>(b.dv + krow * D + i0) = ov;
      *reinterpret_cast<f32x4*>(b.dk + krow * D + i0) = ok;
    }
}

// Memory-update part of dK, dV for the delta rule (k_bwd_update_mfma, Eq. 9 differentiated;
// formulas in backward.hip; the linear rule's part runs in k_bwd_dkv_mfma's epilogue): one
// workgroup = 4 waves = 128 tokens of one segment; every wave owns 32 tokens on lanes, with
// the feature dimension in the result registers:
//   Y^T = G_s^T sigma(K)^T                      (-> dV)
//   R^T = M_{s-1}^T sigma(K)^T / denk,  dsigma(K)^T = G_s (V - R)^T + M_{s-1} dW^T + z ddenk
//   with dW = -Y / denk, ddenk = Y . R / denk (per token)
// G_s (fp32) and M_{s-1} are staged in LDS as bf16 in both orientations (16-row-group
// layout); sigma(K) and V come from registers; the (V - R) and dW results are the B operands
// of the last products, with G_s and M_{s-1} read in the order their registers hold.  dV, dK
// are updated in place (fp32); the tile's sigma(K)^T ddenk partial goes to cpart and the z
// term is added by a later pass.
template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void k_bwd_update_mfma(const BackwardArgs b) {
  constexpr int KS = D / 16, DB = D / 32, CPR = D / 8, DD = D * D;
  // G_s^T (rows j), G_s (rows i), M_{s-1}^T (rows j), M_{s-1} (rows i); once the products
  // are done, the first half holds the tile's per-token sigma(k_t) ddenk_t rows (fp32)
  __shared__ __align__(16) uint16_t lds[4 * DD];
  uint16_t* gt_l = lds;
  uint16_t* gr_l = lds + DD;
  uint16_t* mt_l = lds + 2 * DD;
  uint16_t* mr_l = lds + 3 * DD;
  float* crow = reinterpret_cast<float*>(lds);   // [128 tokens][D]
  static_assert(128 * D * 4 <= 4 * DD * 2, "the per-token rows fit in the staging area");

  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.ct, tile = static_cast<int>(blockIdx.x) % b.ct;
  const int BH = w.B * w.H;
  const int s_local = u / BH, bh = u % BH;
  const int n = w.seg_tokens(s_local);
  const int t0 = tile * 128;
  if (t0 >= n) {   // a tile past a short segment's end: its sigma(K)^T ddenk partial is zero
    if (threadIdx.x < D) b.cpart[(static_cast<int64_t>(u) * b.ct + tile) * D + threadIdx.x] = 0.f;
    return;
  }
  const int64_t row0 = static_cast<int64_t>(bh) * w.T + static_cast<int64_t>(w.s0 + s_local) * w.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  // ---- stage G_s (and M_{s-1}) as bf16 in both orientations
  pack_g<D>(b.gm + static_cast<int64_t>(u) * DD, gr_l, gt_l, tid, kBwdThreads);
  const uint16_t* mt = static_cast<const uint16_t*>(w.ws.mt) + static_cast<int64_t>(u) * DD;
  for (int e = tid; e < D * CPR; e += kBwdThreads) {
    {  // M^T rows (as recorded): chunk (j, ci)
      const int j = e / CPR, ci = e % CPR;
      st16(mt_l + rg_index(j, 8 * ci, CPR), ld16(mt + j * D + 8 * ci));
    }
    {  // M rows: chunk (i, cj) = M^T[8 cj .. + 7][i]
      const int i = e % D, cj = e / D;
      uint16_t x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = mt[(8 * cj + k) * D + i];
      st16(mr_l + rg_index(i, 8 * cj, CPR),
           u32x4{x[0] | (uint32_t(x[1]) << 16), x[2] | (uint32_t(x[3]) << 16), x[4] | (uint32_t(x[5]) << 16),
                 x[6] | (uint32_t(x[7]) << 16)});
    }
  }
  __syncthreads();

  // Token rows are read and written through buffer resources that end at the segment's
  // last token: lanes past it load zeros and their stores are dropped, so no load sits
  // behind a per-lane branch (which would serialise them).
  const int t = t0 + 32 * wave + l32;
  const bool live = t < n;
  const uint32_t nb = static_cast<uint32_t>(n) * D;   // elements of the segment
  const auto krs = buffer_rsrc(static_cast<const uint16_t*>(w.k) + row0 * D, nb * 2);
  const auto vrs = buffer_rsrc(static_cast<const uint16_t*>(w.v) + row0 * D, nb * 2);
  const auto dvrs = buffer_rsrc(b.dv + row0 * D, nb * 4);
  const auto dkrs = buffer_rsrc(b.dk + row0 * D, nb * 4);
  const uint32_t e0 = static_cast<uint32_t>(t) * D;   // this lane's first element
  const float* zb = w.ws.zb + static_cast<int64_t>(u) * D;

  // sigma(k) of this lane's token as the B operand (k = i natural), and sigma(k) . z
  u32x4 kraw[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kraw[ks] = buffer_ld16(krs, 2 * (e0 + 16 * ks + 8 * hl));
  bf16x8 wreg[KS];
  float wf[KS][8];
  float zs = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = elu_plus_one(bf16lo_to_f32(kraw[ks][e])), hi = elu_plus_one(bf16hi_to_f32(kraw[ks][e]));
      wf[ks][2 * e] = live ? lo : 0.f;
      wf[ks][2 * e + 1] = live ? hi : 0.f;
    }
    wreg[ks] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(wf[ks][0], wf[ks][1]), pack_bf16x2(wf[ks][2], wf[ks][3]),
                                               pack_bf16x2(wf[ks][4], wf[ks][5]), pack_bf16x2(wf[ks][6], wf[ks][7])});
#pragma unroll
    for (int e = 0; e < 8; ++e) zs = fmaf(wf[ks][e], zb[16 * ks + 8 * hl + e], zs);
  }
  const int g_rd = ((l32 >> 4) * 16 * CPR + 16 * hl + (l32 & 15)) * 8;
  const int p_rd = ((l32 >> 4) * 16 * CPR + (l32 & 15)) * 8 + 4 * hl;

  f32x16 Y[DB], S[DB];
#pragma unroll
  for (int jb = 0; jb < DB; ++jb) {
    Y[jb] = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      Y[jb] = mfma32x32x16(as_bf16x8(ld16(gt_l + g_rd + jb * 256 * CPR + 256 * ks)), wreg[ks], Y[jb]);
  }
  float ddk;   // ddenk of this lane's token
  {
    const float denk = sum_across_halves(zs) + w.eps;
    const float inv = 1.f / denk;
    f32x16 R[DB];
#pragma unroll
    for (int jb = 0; jb < DB; ++jb) {
      R[jb] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        R[jb] = mfma32x32x16(as_bf16x8(ld16(mt_l + g_rd + jb * 256 * CPR + 256 * ks)), wreg[ks], R[jb]);
    }
    // register r of block jb holds feature j = 32 jb + 8 (r / 4) + 4 hl + r % 4 of this token
    u32x2 vraw[DB][4];
#pragma unroll
    for (int jb = 0; jb < DB; ++jb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) vraw[jb][r4] = buffer_ld8(vrs, 2 * (e0 + 32 * jb + 8 * r4 + 4 * hl));
    float yr = 0.f;
    bf16x8 vrb[KS], dwb[KS];
#pragma unroll
    for (int jb = 0; jb < DB; ++jb) {
      float vmr[16], dw[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const u32x2 vv = vraw[jb][r4];
        const float vf[4] = {bf16lo_to_f32(vv[0]), bf16hi_to_f32(vv[0]), bf16lo_to_f32(vv[1]), bf16hi_to_f32(vv[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float rv = R[jb][r] * inv;
          yr = fmaf(Y[jb][r], rv, yr);
          vmr[r] = vf[e] - rv;
          dw[r] = -Y[jb][r] * inv;
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        vrb[2 * jb + half] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(vmr[8 * half], vmr[8 * half + 1]), pack_bf16x2(vmr[8 * half + 2], vmr[8 * half + 3]),
                          pack_bf16x2(vmr[8 * half + 4], vmr[8 * half + 5]),
                          pack_bf16x2(vmr[8 * half + 6], vmr[8 * half + 7])});
        dwb[2 * jb + half] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(dw[8 * half], dw[8 * half + 1]), pack_bf16x2(dw[8 * half + 2], dw[8 * half + 3]),
                          pack_bf16x2(dw[8 * half + 4], dw[8 * half + 5]), pack_bf16x2(dw[8 * half + 6], dw[8 * half + 7])});
      }
    }
    ddk = sum_across_halves(yr) * inv;
#pragma unroll
    for (int ib = 0; ib < DB; ++ib) {
      S[ib] = zero16();
#pragma unroll
      for (int j4 = 0; j4 < KS; ++j4) {
        const uint16_t* pg = gr_l + p_rd + ib * 256 * CPR + 256 * j4;
        const u32x2 g0 = ld8(pg), g1 = ld8(pg + 128);
        S[ib] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]}), vrb[j4], S[ib]);
        const uint16_t* pm = mr_l + p_rd + ib * 256 * CPR + 256 * j4;
        const u32x2 m0 = ld8(pm), m1 = ld8(pm + 128);
        S[ib] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]}), dwb[j4], S[ib]);
      }
    }
  }
  // this tile's share of sigma(K)^T ddenk (wf and ddk are zero past the segment's end):
  // every token's row sigma(k_t) ddenk_t goes to LDS once all waves are done with the
  // staged G_s and M_{s-1}, and is summed over the tile's tokens in token order (no
  // atomics: the result does not depend on the order in which the waves arrive)
  __syncthreads();
  {
    float* cr = crow + (32 * wave + l32) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = wf[ks][e] * ddk;
        hi[e] = wf[ks][4 + e] * ddk;
      }
      *reinterpret_cast<f32x4*>(cr + 16 * ks) = lo;
      *reinterpret_cast<f32x4*>(cr + 16 * ks + 4) = hi;
    }
  }
  // dV += Y (all loads of a block first, then the stores)
#pragma unroll
  for (int jb = 0; jb < DB; ++jb) {
    u32x4 old[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) old[r4] = buffer_ld16(dvrs, 4 * (e0 + 32 * jb + 8 * r4 + 4 * hl));
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(__uint_as_float(old[r4][e]) + Y[jb][4 * r4 + e]);
      buffer_st16(dvrs, 4 * (e0 + 32 * jb + 8 * r4 + 4 * hl), o);
    }
  }
  // dK += dsigma(K) o sigma'(K)
#pragma unroll
  for (int ib = 0; ib < DB; ++ib) {
    u32x4 old[4];
    u32x2 kv[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      old[r4] = buffer_ld16(dkrs, 4 * (e0 + 32 * ib + 8 * r4 + 4 * hl));
      kv[r4] = buffer_ld8(krs, 2 * (e0 + 32 * ib + 8 * r4 + 4 * hl));
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int i0 = 32 * ib + 8 * r4 + 4 * hl;
      const float kf[4] = {bf16lo_to_f32(kv[r4][0]), bf16hi_to_f32(kv[r4][0]), bf16lo_to_f32(kv[r4][1]),
                           bf16hi_to_f32(kv[r4][1])};
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = S[ib][4 * r4 + e];
        a = fmaf(ddk, zb[i0 + e], a);
        o[e] = __float_as_uint(__uint_as_float(old[r4][e]) +
                               a * (kf[e] > 0.f ? 1.f : __builtin_amdgcn_exp2f(kf[e] * kLog2e)));
      }
      buffer_st16(dkrs, 4 * (e0 + i0), o);
    }
  }
  __syncthreads();
  if (tid < D) {
    float c = 0.f;
#pragma unroll 8
    for (int r = 0; r < 128; ++r) c += crow[r * D + tid];
    b.cpart[(static_cast<int64_t>(u) * b.ct + tile) * D + tid] = c;
  }
}

// R_s = sigma(Q)^T dnum and r_s = sigma(Q)^T dden over one chunk of a segment (dnum = g dO /
// den), the retrieval's contribution to dL/dM_{s-1} and dL/dz_{s-1}: the contraction runs
// over tokens, so both operands are read from 64-token LDS tiles ([token][d], 16-row
// groups) by transpose reads; the d x d result is spread over the 4 waves.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_r_mfma(const BackwardArgs b) {
  constexpr int DB = D / 32, CPR = D / 8, SUB = 64;
  constexpr int NBW = DB * DB / 4;          // 32 x 32 result blocks per wave
  constexpr int PH = kBwdThreads / CPR;     // row phases of the tile loads
  __shared__ __align__(16) uint16_t sq_l[SUB * D];
  __shared__ __align__(16) uint16_t dn_l[SUB * D];
  __shared__ float rz_l[PH][D];
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.rch, ch = static_cast<int>(blockIdx.x) % b.rch;
  const int BH = w.B * w.H;
  const int s_local = u / BH, bh = u % BH, h = bh % w.H;
  const int n = w.seg_tokens(s_local);
  const int64_t row0 = static_cast<int64_t>(bh) * w.T + static_cast<int64_t>(w.s0 + s_local) * w.N;
  const int per = (w.N + b.rch - 1) / b.rch;
  const int t_lo = ch * per, t_hi = min(n, t_lo + per);
  const float g = w.gate_g[h];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int G = lane >> 4, jl = lane & 15;
  const int m_rd = (16 * (2 * (G & 1) + ((jl & 3) >> 1)) + 8 * (G >> 1) + (jl >> 2)) * 8 + 4 * (jl & 1);
  (void)l32;

  f32x16 acc[NBW];
#pragma unroll
  for (int k = 0; k < NBW; ++k) acc[k] = zero16();
  float rzp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rzp[e] = 0.f;
  const int cl = tid % CPR, rp = tid / CPR;   // this thread's chunk (columns 8 cl ..) and row phase
  const uint16_t* qg = static_cast<const uint16_t*>(w.q);
  const uint16_t* og = static_cast<const uint16_t*>(b.dout);

  // The rows of a 64-token tile: this thread's RPS rows of Q and dO (16 bytes each) and their
  // den, dden, loaded with no per-lane branch (rows past the chunk end re-read its last row and
  // are zeroed when used) one tile ahead of their use, so the loads never wait behind one another.
  constexpr int RPS = SUB / PH;
  struct RowSet {
    u32x4 q[RPS], o[RPS];
    float den[RPS], dz[RPS];
  };
  auto fetch = [&](int t0, RowSet& rs) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < RPS; ++p) {
      const int t = min(t0 + p * PH + rp, t_hi - 1);
      const int64_t x = (row0 + t) * D + 8 * cl;
      rs.q[p] = ld16(qg + x);
      rs.o[p] = ld16(og + x);
      rs.den[p] = b.den[row0 + t];
      rs.dz[p] = b.dden[row0 + t];
    }
  };
  auto consume = [&](int t0, const RowSet& rs) __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < RPS; ++p) {
      const int r = p * PH + rp;
      const bool ok = t0 + r < t_hi;
      const float sc = ok ? g / rs.den[p] : 0.f, dz = ok ? rs.dz[p] : 0.f;
      float sv[8], dv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s0 = elu_plus_one(bf16lo_to_f32(rs.q[p][e])), s1 = elu_plus_one(bf16hi_to_f32(rs.q[p][e]));
        sv[2 * e] = ok ? s0 : 0.f;
        sv[2 * e + 1] = ok ? s1 : 0.f;
        dv[2 * e] = bf16lo_to_f32(rs.o[p][e]) * sc;
        dv[2 * e + 1] = bf16hi_to_f32(rs.o[p][e]) * sc;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) rzp[e] = fmaf(sv[e], dz, rzp[e]);
      st16(sq_l + rg_index(r, 8 * cl, CPR), u32x4{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                                                  pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7])});
      st16(dn_l + rg_index(r, 8 * cl, CPR), u32x4{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]),
                                                  pack_bf16x2(dv[4], dv[5]), pack_bf16x2(dv[6], dv[7])});
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < SUB / 16; ++ks) {
#pragma unroll
      for (int k = 0; k < NBW; ++k) {
        const int blk = wave * NBW + k, ib = blk / DB, jb = blk % DB;
        const uint16_t* pa = sq_l + m_rd + ks * 128 * CPR + ib * 512;
        const uint16_t* pb = dn_l + m_rd + ks * 128 * CPR + jb * 512;
        const u32x2 a0 = lds_read_tr16(pa), a1 = lds_read_tr16(pa + 32);
        const u32x2 b0 = lds_read_tr16(pb), b1 = lds_read_tr16(pb + 32);
        acc[k] = mfma32x32x16(__builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]}),
                              __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]}), acc[k]);
      }
    }
  };
  RowSet ra, rb;
  fetch(t_lo, ra);
  for (int t0 = t_lo; t0 < t_hi; t0 += 2 * SUB) {
    fetch(t0 + SUB, rb);
    consume(t0, ra);
    if (t0 + SUB >= t_hi) break;
    fetch(t0 + 2 * SUB, ra);
    consume(t0 + SUB, rb);
  }
  // R block (ib, jb): register r of lane l holds R[32 ib + 8 (r / 4) + 4 hl + r % 4][32 jb + l % 32]
  float* rpo = b.rpart + (static_cast<int64_t>(u) * b.rch + ch) * D * D;
  const int hl = lane >> 5;
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    const int blk = wave * NBW + k, ib = blk / DB, jb = blk % DB;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      rpo[(32 * ib + 8 * (r >> 2) + 4 * hl + (r & 3)) * D + 32 * jb + (lane & 31)] = acc[k][r];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) rz_l[rp][8 * cl + e] = rzp[e];
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int p = 0; p < PH; ++p) a += rz_l[p][tid];
    b.rzpart[(static_cast<int64_t>(u) * b.rch + ch) * D + tid] = a;
  }
}

}  // namespace

hipError_t launch_bwd_r_mfma(const BackwardArgs& b, hipStream_t st) {
  const WindowArgs& w = b.w;
  const dim3 grid(static_cast<unsigned>(w.units() * b.rch)), block(kBwdThreads);
  if (w.D == 128) hipLaunchKernelGGL((k_bwd_r_mfma<128>), grid, block, 0, st, b);
  else if (w.D == 64) hipLaunchKernelGGL((k_bwd_r_mfma<64>), grid, block, 0, st, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_update_mfma(const BackwardArgs& b, hipStream_t st) {
  const WindowArgs& w = b.w;
  const dim3 grid(static_cast<unsigned>(w.units() * b.ct)), block(kBwdThreads);
  if (!w.delta) return hipErrorInvalidValue;   // (linear: fused into the dK, dV kernel)
  if (w.D == 128) hipLaunchKernelGGL((k_bwd_update_mfma<128>), grid, block, 0, st, b);
  else if (w.D == 64) hipLaunchKernelGGL((k_bwd_update_mfma<64>), grid, block, 0, st, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkv_mfma(const BackwardArgs& b, bool fuse_update, hipStream_t st) {
  const WindowArgs& w = b.w;
  // the fused epilogue takes sigma(K) from the local arm's keys and G_s from gpk
  if (fuse_update && (w.delta || w.k_loc != w.k || !b.gpk)) return hipErrorInvalidValue;
  const int nk = (w.N + kBwdQ - 1) / kBwdQ;
  const dim3 grid(static_cast<unsigned>(w.units() * nk)), block(kBwdThreads);
  if (w.D == 128) {
    if (fuse_update) hipLaunchKernelGGL((k_bwd_dkv_mfma<128, true>), grid, block, 0, st, b);
    else hipLaunchKernelGGL((k_bwd_dkv_mfma<128, false>), grid, block, 0, st, b);
  } else if (w.D == 64) {
    if (fuse_update) hipLaunchKernelGGL((k_bwd_dkv_mfma<64, true>), grid, block, 0, st, b);
    else hipLaunchKernelGGL((k_bwd_dkv_mfma<64, false>), grid, block, 0, st, b);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_gpack(const BackwardArgs& b, hipStream_t st) {
  const WindowArgs& w = b.w;
  if (!b.gpk) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(w.units())), block(kBwdThreads);
  if (w.D == 128) hipLaunchKernelGGL((k_bwd_gpack<128>), grid, block, 0, st, b);
  else if (w.D == 64) hipLaunchKernelGGL((k_bwd_gpack<64>), grid, block, 0, st, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq_mfma(const BackwardArgs& b, hipStream_t st) {
  const WindowArgs& w = b.w;
  const int nq = (w.N + kBwdQ - 1) / kBwdQ;
  const dim3 grid(static_cast<unsigned>(w.units() * nq)), block(kBwdThreads);
  if (w.D == 128) hipLaunchKernelGGL((k_bwd_dq_mfma<128>), grid, block, 0, st, b);
  else if (w.D == 64) hipLaunchKernelGGL((k_bwd_dq_mfma<64>), grid, block, 0, st, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace infini
