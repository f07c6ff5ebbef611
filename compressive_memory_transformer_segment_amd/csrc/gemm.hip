// Dense projections around the Infini-attention layer ("Leave No Context Behind",
// arXiv 2404.07143, section 3.1): Q = X W_Q, K = X W_K, V = X W_V (Eq. 5) and the
// multi-head output O = [A_1; ...; A_H] W_O (Eq. 11).  One bf16 MFMA kernel computes
// C = A W^T with a row map for A and a column map for C, so it reads the per-head
// attention output and writes per-head Q / K / V in the [B, H, T, d] layout the attention
// kernels use, without separate transpose passes.
//
// Tiling (gfx950): a workgroup = 8 waves (two per SIMD, so one wave's waits are covered
// by the other's products) computes a 256-token x 256-feature tile; each wave owns 128
// features x 64 tokens of it, 8 MFMA 32x32x16 accumulators (128 registers).
// The MFMAs run in the transposed frame, D[n][t] = (W A^T)[n][t]: a lane then holds one
// token and four consecutive output features in each result register quad, which become
// one 8-byte store.  Both operands go HBM -> LDS by buffer -> LDS copies in stages of 32 k,
// four buffers deep (stage s + 3 is in flight while stage s is consumed), into the
// row-group layout: 1 KB copy = 16 rows x 64 bytes, chunk c (8 values) of row r in slot
// (r / 16) * 64 + 16 c + r % 16.  Every MFMA operand read is then a conflict-free
// ds_read_b128 at an immediate offset from one base register.  There is one barrier per
// stage, in the middle of the stage's MFMAs, so the operand reads of the next stage are
// issued while the current stage's products run.
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kWaves = 8;                     // 2 per SIMD
constexpr int kGT = 64 * kWaves;
constexpr int kGM = 256;                      // tokens per tile
constexpr int kGN = 256;                      // output features per tile
constexpr int kGK = 32;                       // k per stage
constexpr int kStage = (kGN + kGM) * kGK;     // elements of one buffer: [W tile | A tile]
constexpr int kGroupM = 2;                    // token tiles per group of the tile order
constexpr int kWN = 2;                        // waves along the features
constexpr int kWM = kWaves / kWN;             // waves along the tokens
constexpr int kTI = kGN / kWN / 32;           // 32-feature blocks per wave
constexpr int kTJ = kGM / kWM / 32;           // 32-token blocks per wave
constexpr int kCPW = 16 / kWaves;             // row groups of each operand a wave copies per stage
static_assert(kCPW * kWaves == 16 && kTI * kWN * 32 == kGN && kTJ * kWM * 32 == kGM, "tile split");

template <int N_>
using IC = std::integral_constant<int, N_>;

// Workgroup -> (token tile, feature tile).  Block b runs on XCD b % 8; XCD x takes a
// contiguous range of the tile order, in which groups of kGroupM token tiles run over all
// feature tiles, so the A and W rows that one XCD's workgroups read at a time are few and
// are shared through its L2.
__device__ __forceinline__ void gemm_tile(int MT, int NT, int& mt, int& nt) {
  const int P = MT * NT;
  const int bid = static_cast<int>(blockIdx.x);
  const int x = bid % 8, j = bid / 8;
  const int per = P / 8, extra = P % 8;
  const int t = x * per + min(x, extra) + j;
  const int g = t / (kGroupM * NT);
  const int first = g * kGroupM;
  const int gm = min(kGroupM, MT - first);
  const int r = t - g * kGroupM * NT;
  mt = first + r % gm;
  nt = r / gm;
}


__global__ __launch_bounds__(kGT, 1) void k_gemm(const GemmArgs g) {
  __shared__ __align__(16) uint16_t buf0[kStage];
  __shared__ __align__(16) uint16_t buf1[kStage];
  __shared__ __align__(16) uint16_t buf2[kStage];
  __shared__ __align__(16) uint16_t buf3[kStage];

  const int TT = (g.T + kGM - 1) / kGM;
  int mt, nt;
  gemm_tile(g.nb * TT, (g.N + kGN - 1) / kGN, mt, nt);
  const int b = mt / TT;
  const int t0 = (mt - b * TT) * kGM, n0 = nt * kGN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wn = wave % kWN, wm = wave / kWN;   // the wave's features / tokens
  const int S = g.K / kGK;

  // copies: wave w fills row groups kCPW w .. kCPW w + kCPW - 1 of the W tile and of the A tile; lane i
  // takes row 16 grp + i % 16, chunk i / 16 of the stage.  One buffer resource per operand
  // starts at row 0 of the tile at the stage's first k and spans the valid rows (rows past
  // the end read as zeros); the row group is in the lane offset.
  const int64_t K2 = static_cast<int64_t>(g.K) * 2, a_st2 = g.a_st * 2;
  const char* wcur = static_cast<const char*>(g.w) + n0 * K2;
  const char* acur = static_cast<const char*>(g.a) + (b * g.a_sb + static_cast<int64_t>(t0) * g.a_st) * 2;
  int a_kk = 0;   // k of the next stage within its a_dk block
  const int w_rows = min(g.N - n0, kGN), a_rows = min(g.T - t0, kGM);
  const uint32_t w_bytes = static_cast<uint32_t>((w_rows - 1) * K2 + 64);
  const uint32_t a_bytes = static_cast<uint32_t>((a_rows - 1) * a_st2 + 64);
  uint32_t vo_w[kCPW], vo_a[kCPW];
#pragma unroll
  for (int j = 0; j < kCPW; ++j) {
    const int r = 16 * (kCPW * wave + j) + (lane & 15);
    vo_w[j] = static_cast<uint32_t>(r * K2) + 16 * (lane >> 4);
    vo_a[j] = static_cast<uint32_t>(r * a_st2) + 16 * (lane >> 4);
  }

  auto bufp = [&](auto bc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int bi = decltype(bc)::value & 3;
    if constexpr (bi == 0) return buf0;
    else if constexpr (bi == 1) return buf1;
    else if constexpr (bi == 2) return buf2;
    else return buf3;
  };
  // the next stage (stages are issued in order, k = 32 s .. 32 s + 31) into dst: 8 copy
  // instructions per wave.  Stages past the end are issued too, as zero fills, so that
  // every stage is 8 copies and the waits are constants.
  int s_next = 0;
  auto issue = [&](uint16_t* dst) __attribute__((always_inline)) {
    const bool live = s_next < S;
    ++s_next;
#pragma unroll
    for (int j = 0; j < kCPW; ++j) copy_to_lds(wcur, live ? w_bytes : 0u, dst + 512 * (kCPW * wave + j), vo_w[j]);
#pragma unroll
    for (int j = 0; j < kCPW; ++j)
      copy_to_lds(acur, live ? a_bytes : 0u, dst + kGN * kGK + 512 * (kCPW * wave + j), vo_a[j]);
    if (live) {
      wcur += 2 * kGK;
      acur += 2 * kGK;
      a_kk += kGK;
      if (a_kk == g.a_dk) {   // next block of the A column map
        a_kk = 0;
        acur += 2 * (g.a_sh - g.a_dk);
      }
    }
  };

  // operand reads: row 32 blk + l32 of the wave's rows, chunk 2 ks + hl
  const int rd = ((l32 >> 4) * 64 + 16 * hl + (l32 & 15)) * 8;
  const int rw = kTI * 1024 * wn + rd, ra = kGN * kGK + kTJ * 1024 * wm + rd;

  f32x16 acc[kTI][kTJ];
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j) acc[i][j] = zero16();
  bf16x8 fa0[kTI], fb0[kTJ], fa1[kTI], fb1[kTJ];

  auto load = [&](const uint16_t* buf, int ks, bf16x8 (&fa)[kTI], bf16x8 (&fb)[kTJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTI; ++i) fa[i] = as_bf16x8(ld16(buf + rw + 1024 * i + 256 * ks));
#pragma unroll
    for (int j = 0; j < kTJ; ++j) fb[j] = as_bf16x8(ld16(buf + ra + 1024 * j + 256 * ks));
  };
  auto mma = [&](const bf16x8 (&fa)[kTI], const bf16x8 (&fb)[kTJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTI; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
  };
  // the operand reads of the next half go out one by one between the first products
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTI + kTJ; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kTI * kTJ - kTI - kTJ, 0);
  };
  // stage s from buffer s % 4; its first half's operands are already in fa0 / fb0
  auto step = [&](auto bc, int s) __attribute__((always_inline)) {
    constexpr int bi = decltype(bc)::value;
    load(bufp(IC<bi>{}), 1, fa1, fb1);
    mma(fa0, fb0);
    interleave();
    wait_vm_lgkm0<2 * kCPW>();      // this wave's copies of stage s + 1 have landed
    __builtin_amdgcn_s_barrier();   // ... everyone's; and everyone is done with stage s - 1
    issue(bufp(IC<bi + 3>{}));   // stage s + 3
    load(bufp(IC<bi + 1>{}), 0, fa0, fb0);   // (past the last stage: unused)
    mma(fa1, fb1);
    interleave();
  };

  issue(buf0);
  issue(buf1);
  issue(buf2);
  wait_vm_lgkm0<4 * kCPW>();   // stage 0
  __builtin_amdgcn_s_barrier();
  load(buf0, 0, fa0, fb0);
  for (int s = 0; s < S; s += 4) {
    step(IC<0>{}, s);
    if (s + 1 < S) step(IC<1>{}, s + 1);
    if (s + 2 < S) step(IC<2>{}, s + 2);
    if (s + 3 < S) step(IC<3>{}, s + 3);
  }
  wait_vm_lgkm0<0>();   // no copy may land in LDS after the workgroup ends

  // epilogue: register quad q of accumulator (i, j) holds features
  // n0 + 32 (kTI wn + i) + 8 q + 4 hl + 0..3 of token t0 + 32 (kTJ wm + j) + l32
  int64_t trow[kTJ];
  bool tok_ok[kTJ];
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    const int t = t0 + 32 * (kTJ * wm + j) + l32;
    tok_ok[j] = t < g.T;
    trow[j] = b * g.c_sb + static_cast<int64_t>(t) * g.c_st;
  }
#pragma unroll
  for (int i = 0; i < kTI; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nu = n0 + 32 * (kTI * wn + i) + 8 * q;   // wave-uniform
      if (nu >= g.N) continue;
      const int part = nu / g.c_np, rem = nu - part * g.c_np;
      const int hh = rem / g.c_dh, jj = rem - hh * g.c_dh;
      uint16_t* cb = static_cast<uint16_t*>(part == 0 ? g.c[0] : (part == 1 ? g.c[1] : g.c[2])) +
                     hh * g.c_sh + jj + 4 * hl;
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        if (!tok_ok[j]) continue;
        const f32x16& v = acc[i][j];
        st8(cb + trow[j], u32x2{pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3])});
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  const int64_t TT = (static_cast<int64_t>(g.T) + kGM - 1) / kGM;
  const int64_t P = static_cast<int64_t>(g.nb) * TT * ((g.N + kGN - 1) / kGN);
  if (P == 0) return hipSuccess;
  if (P > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm, dim3(static_cast<unsigned>(P)), dim3(kGT), 0, st, g);
  return hipGetLastError();
}

}  // namespace infini
