// The memory chain: the only sequential step of the layer (Eq. 4, "The Recurrent
// Formulation of Infini-Attention", in the architecture summary of arXiv 2404.07143).
//
// Works on M^T ([d_value][d_key]), the layout the retrieval contraction reads:
//   linear (Eq. 8):  M^T_s = M^T_{s-1} + U^T_s
//   delta  (Eq. 9):  M^T_s = M^T_{s-1} - M^T_{s-1} G_s^T + U^T_s   (from M_s = M - G M + U)
//   z_s = z_{s-1} + dz_s
// with U_s, G_s, dz_s from the state pass, which leaves them as per-chunk partials; the
// chain adds the chunks in chunk order.  Rows of M^T (value features) evolve
// independently under both rules, so each workgroup owns a block of rows and never
// waits on another.  For every segment of the window the chain first records the state
// the segment reads (M^T_{s-1} in the attention kernel's operand type, and z_{s-1}), then
// advances it; the window's final state goes back to the handle's M ([d_key][d_value]) and z.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kChainFillWorkgroups = 256;   // below this many 16-row workgroups, use 8 rows

// Linear rule.  A workgroup owns RB rows of M^T (value features rb .. rb + RB - 1) of one
// (b,h); thread (r, cg) owns row rb + r, columns EPT cg .. EPT cg + EPT - 1 (EPT = D / 16),
// so a wave reads four whole rows of every U^T partial.  M ([d_key][d_value]) is read
// and written once per window through an LDS transpose, with 16-byte accesses that cover
// the workgroup's 4 RB-byte pieces of M's rows.  RB = 16 (256 threads), or 8 (128 threads:
// twice the workgroups, for few (b,h) pairs, where each workgroup's stream of partials
// sets the time).
template <int D, int CHK, bool BF16, int RB>
__global__ __launch_bounds__(16 * RB) void k_chain_linear(const WindowArgs a) {
  constexpr int NT = 16 * RB;             // threads
  constexpr int EPT = D / 16;             // elements per thread
  constexpr int CG = D / EPT;             // thread columns per row (16)
  constexpr int TPR = RB / 4;             // threads per row of M in the transposing accesses
  constexpr int RPP = NT / TPR;           // rows of M per pass of those accesses
  constexpr int kBatch = CHK >= 2 ? 16 / CHK : 8;    // segments whose partials are loaded together
  static_assert(RB * CG == NT && D % RPP == 0 && NT >= D, "one thread per (row, column group)");
  __shared__ float tr[D][RB + 1];         // M[i][rb + c] at tr[i][c]
  const int BH = a.B * a.H;
  const int bh = blockIdx.x / (D / RB);
  const int rb = (blockIdx.x % (D / RB)) * RB;
  const int tid = threadIdx.x;
  const int r = tid / CG, cg = tid % CG;
  const int dv = rb + r;
  const int i0 = cg * EPT;
  const int64_t DD = static_cast<int64_t>(D) * D;
  float* Mb = a.M + bh * DD + rb;

  float m[EPT];
  if (a.zero_state) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) m[e] = 0.f;
  } else {
    // thread t: row t / TPR (+ RPP k) of M, columns rb + 4 (t % TPR) .. +3
#pragma unroll
    for (int k = 0; k < D / RPP; ++k) {
      const int i = tid / TPR + RPP * k;
      const f32x4 v = *reinterpret_cast<const f32x4*>(Mb + static_cast<int64_t>(i) * D + 4 * (tid % TPR));
#pragma unroll
      for (int c = 0; c < 4; ++c) tr[i][4 * (tid % TPR) + c] = v[c];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) m[e] = tr[i0 + e][r];
  }
  const bool zown = rb == 0 && tid < D;
  float z = zown && !a.zero_state ? a.z[static_cast<int64_t>(bh) * D + tid] : 0.f;

  for (int s0 = 0; s0 < a.W; s0 += kBatch) {
    // all chunk partials of the batch are independent of the chain: issue them together
    f32x4 ut[kBatch][CHK][EPT / 4];
    float dzv[kBatch][CHK];
#pragma unroll
    for (int sb = 0; sb < kBatch; ++sb) {
      const int s = min(s0 + sb, a.W - 1);
      const int64_t u = static_cast<int64_t>(s) * BH + bh;
#pragma unroll
      for (int c = 0; c < CHK; ++c) {
        const int64_t slot = u * CHK + c;
        const float* src = a.ws.u + slot * DD + static_cast<int64_t>(dv) * D + i0;
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) ut[sb][c][q] = *reinterpret_cast<const f32x4*>(src + 4 * q);
        // every thread loads (threads past D re-read the first D; only owners use them):
        // a load under the owner test made the compiler wait for each one before the next
        dzv[sb][c] = a.ws.dz[slot * D + (tid & (D - 1))];
      }
    }
#pragma unroll
    for (int sb = 0; sb < kBatch; ++sb) {
      const int s = s0 + sb;
      if (s >= a.W) break;
      const int64_t u = static_cast<int64_t>(s) * BH + bh;
      const int64_t off = u * DD + static_cast<int64_t>(dv) * D + i0;
      if constexpr (BF16) {
        uint16_t* mt = static_cast<uint16_t*>(a.ws.mt) + off;
        uint32_t pk[EPT / 2];
#pragma unroll
        for (int e = 0; e < EPT / 2; ++e) pk[e] = pack_bf16x2(m[2 * e], m[2 * e + 1]);
        if constexpr (EPT == 8) {
          st16(mt, u32x4{pk[0], pk[1], pk[2], pk[3]});
        } else {
          st8(mt, u32x2{pk[0], pk[1]});
        }
      } else {
        float* mt = static_cast<float*>(a.ws.mt) + off;
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) *reinterpret_cast<f32x4*>(mt + 4 * q) = f32x4{m[4 * q], m[4 * q + 1], m[4 * q + 2], m[4 * q + 3]};
      }
      if (zown) {
        a.ws.zb[u * D + tid] = z;
        float dz = 0.f;
#pragma unroll
        for (int c = 0; c < CHK; ++c) dz += dzv[sb][c];
        z += dz;
      }
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float add = 0.f;
#pragma unroll
        for (int c = 0; c < CHK; ++c) add += ut[sb][c][e / 4][e % 4];
        m[e] += add;
      }
    }
  }
  if (BF16 && a.mt_cur) {   // the final state as the retrieval operand of the next call
    uint16_t* mc = static_cast<uint16_t*>(a.mt_cur) + bh * DD + static_cast<int64_t>(dv) * D + i0;
    uint32_t pk[EPT / 2];
#pragma unroll
    for (int e = 0; e < EPT / 2; ++e) pk[e] = pack_bf16x2(m[2 * e], m[2 * e + 1]);
    if constexpr (EPT == 8) {
      st16(mc, u32x4{pk[0], pk[1], pk[2], pk[3]});
    } else {
      st8(mc, u32x2{pk[0], pk[1]});
    }
  }
  if (zown) {
    a.z[static_cast<int64_t>(bh) * D + tid] = z;
    if (a.z_cur) a.z_cur[static_cast<int64_t>(bh) * D + tid] = z;
  }
  __syncthreads();   // every thread is past its reads of tr
#pragma unroll
  for (int e = 0; e < EPT; ++e) tr[i0 + e][r] = m[e];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < D / RPP; ++k) {
    const int i = tid / TPR + RPP * k;
    f32x4 v;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = tr[i][4 * (tid % TPR) + c];
    *reinterpret_cast<f32x4*>(Mb + static_cast<int64_t>(i) * D + 4 * (tid % TPR)) = v;
  }
}

// Delta rule, G_s summed over the chunks beforehand (k_gsum).  A workgroup owns R = 4 RPT
// rows of M^T of one (b,h); thread (g, i) owns rows rb + RPT g .. + RPT - 1, column i (g is
// wave-uniform, so the reads of M^T rows are broadcasts; thread i reads row i of G_s once
// per step for its RPT rows).  Nothing but M^T itself depends on the chain, so step s + 1's G
// and U^T / key-sum partials are loaded into registers while step s multiplies, and G_{s+1}
// is staged into the other of two LDS buffers at the end of step s.  One barrier per step.
// Two waves per SIMD, so that one wave's LDS latency is covered by the other's FMAs.  Rows of
// M^T evolve independently, so workgroups never wait on each other.  Every workgroup stages
// all of G_s each step: more rows per workgroup (RPT = 4) divide that traffic by four when
// there are enough (b,h) pairs to fill the compute units with fewer workgroups.
template <int D, int CHK, bool BF16, int RPT>
__global__ __launch_bounds__(4 * D, 1) void k_chain_delta(const WindowArgs a, const float* __restrict__ gsum) {
  constexpr int NT = 4 * D;
  constexpr int R = 4 * RPT;              // rows of M^T per workgroup
  constexpr int GP = D + 4;               // LDS row pitch of G and of the M^T rows (floats)
  constexpr int GV = D * D / 4 / NT;      // float4 elements of G_s per thread
  constexpr int MPT = R * D / NT;         // elements of M per thread in the transposing loads (RPT)
  __shared__ __align__(16) float g_lds[2][D][GP];
  __shared__ __align__(16) float m_lds[2][R][GP];

  const int BH = a.B * a.H;
  const int W = a.W;
  const int bh = blockIdx.x / (D / R);
  const int rb = (blockIdx.x % (D / R)) * R;
  const int tid = threadIdx.x;
  const int g = tid / D, i = tid % D;     // g is wave-uniform (D is a multiple of 64)
  const int r0 = RPT * g;                 // this thread's first row in the workgroup's block
  const int64_t DD = static_cast<int64_t>(D) * D;

  // M^T[rb + r][i] = M[i][rb + r]: the workgroup's R columns of M through LDS (thread t reads
  // MPT consecutive columns of row t / (R / MPT))
  float* Mb = a.M + bh * DD + rb;
  const int mrow = tid / (R / MPT), mcol = (tid % (R / MPT)) * MPT;
  float m[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) m[j] = 0.f;
  if (!a.zero_state) {
    const float* src = Mb + static_cast<int64_t>(mrow) * D + mcol;
    if constexpr (MPT == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
      for (int c = 0; c < 4; ++c) m_lds[0][mcol + c][mrow] = v[c];
    } else {
#pragma unroll
      for (int c = 0; c < MPT; ++c) m_lds[0][mcol + c][mrow] = src[c];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RPT; ++j) m[j] = m_lds[0][r0 + j][i];
  }
  const bool zown = rb == 0 && tid < D;
  float z = zown && !a.zero_state ? a.z[static_cast<int64_t>(bh) * D + tid] : 0.f;

  // what one step loads ahead of the chain
  struct Pre {
    f32x4 g[GV];
    float up[CHK][RPT];
    float dz[CHK];
  };
  auto fetch = [&](int s, Pre& p) __attribute__((always_inline)) {
    const int64_t u = static_cast<int64_t>(min(s, W - 1)) * BH + bh;
    const float* src = gsum + u * DD;
#pragma unroll
    for (int v = 0; v < GV; ++v) p.g[v] = *reinterpret_cast<const f32x4*>(src + 4 * (tid + v * NT));
#pragma unroll
    for (int c = 0; c < CHK; ++c) {
#pragma unroll
      for (int j = 0; j < RPT; ++j)
        p.up[c][j] = a.ws.u[(u * CHK + c) * DD + static_cast<int64_t>(rb + r0 + j) * D + i];
      p.dz[c] = a.ws.dz[(u * CHK + c) * D + i];   // used by owners only
    }
  };
  auto stage = [&](int b, const Pre& p) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < GV; ++v) {
      const int e = 4 * (tid + v * NT);
      *reinterpret_cast<f32x4*>(&g_lds[b][e / D][e % D]) = p.g[v];
    }
  };
  // step s of the chain: p holds step s's partials, G_s is in LDS buffer s % 2, and nx
  // holds step s + 1's loads (its G is staged at the end)
  auto step = [&](int s, const Pre& p, const Pre& nx) __attribute__((always_inline)) {
    const int b = s & 1;
    const int64_t u = static_cast<int64_t>(s) * BH + bh;
    // record the state this segment reads
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int64_t off = u * DD + static_cast<int64_t>(rb + r0 + j) * D + i;
      if constexpr (BF16) static_cast<uint16_t*>(a.ws.mt)[off] = f32_to_bf16(m[j]);
      else static_cast<float*>(a.ws.mt)[off] = m[j];
      m_lds[b][r0 + j][i] = m[j];
    }
    if (zown) {
      a.ws.zb[u * D + tid] = z;
      float dz = 0.f;
#pragma unroll
      for (int c = 0; c < CHK; ++c) dz += p.dz[c];
      z += dz;
    }
    __syncthreads();   // G_s and this step's rows of M^T are in LDS
    // (M^T G^T)[row][i] = sum_k M^T[row][k] G[i][k], as four interleaved partial sums
    // (k mod 4) per row; k in blocks of 16 whose G reads serve all RPT rows
    f32x4 acc[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int kk = 0; kk < D; kk += 16) {
      f32x4 gk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) gk[q] = *reinterpret_cast<const f32x4*>(&g_lds[b][i][kk + 4 * q]);
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        f32x4 mk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) mk[q] = *reinterpret_cast<const f32x4*>(&m_lds[b][r0 + j][kk + 4 * q]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j][e] = fmaf(mk[q][e], gk[q][e], acc[j][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      float ut = 0.f;
#pragma unroll
      for (int c = 0; c < CHK; ++c) ut += p.up[c][j];
      m[j] = (m[j] - ((acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]))) + ut;
    }
    // G_{s+1} into the buffer step s - 1 read (every thread is past this step's barrier)
    stage(b ^ 1, nx);
  };

  // two register sets: step s's partials in one, step s + 1's loads in the other
  if (W > 0) {
    Pre pa, pb;
    fetch(0, pa);
    stage(0, pa);
    for (int s = 0; s < W; s += 2) {
      fetch(s + 1, pb);
      step(s, pa, pb);
      if (s + 1 < W) {
        fetch(s + 2, pa);
        step(s + 1, pb, pa);
      }
    }
  }
  if (zown) {
    a.z[static_cast<int64_t>(bh) * D + tid] = z;
    if (a.z_cur) a.z_cur[static_cast<int64_t>(bh) * D + tid] = z;
  }
  if (BF16 && a.mt_cur)   // the final state as the retrieval operand of the next call
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      static_cast<uint16_t*>(a.mt_cur)[bh * DD + static_cast<int64_t>(rb + r0 + j) * D + i] = f32_to_bf16(m[j]);
  __syncthreads();   // every thread is past the last step's reads of m_lds
#pragma unroll
  for (int j = 0; j < RPT; ++j) m_lds[0][r0 + j][i] = m[j];
  __syncthreads();
  {
    float* dst = Mb + static_cast<int64_t>(mrow) * D + mcol;
    if constexpr (MPT == 4) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = m_lds[0][mcol + c][mrow];
      *reinterpret_cast<f32x4*>(dst) = v;
    } else {
#pragma unroll
      for (int c = 0; c < MPT; ++c) dst[c] = m_lds[0][mcol + c][mrow];
    }
  }
}

// M [pairs][D][D] (fp32, [d_key][d_value]) -> M^T in bf16 ([d_value][d_key]), through a
// 32 x 32 LDS tile: the retrieval operand of a state set from outside.
template <int D>
__global__ __launch_bounds__(256) void k_state_to_mt(const float* __restrict__ M, uint16_t* __restrict__ mt) {
  __shared__ float tile[32][33];
  constexpr int TB = D / 32;
  const int64_t pair = blockIdx.x / (TB * TB);
  const int tb = blockIdx.x % (TB * TB), ti = (tb / TB) * 32, tj = (tb % TB) * 32;   // rows of M, columns of M
  const float* src = M + pair * D * D;
  uint16_t* dst = mt + pair * D * D;
  const int x = threadIdx.x % 32, y = threadIdx.x / 32;
#pragma unroll
  for (int r = y; r < 32; r += 8) tile[r][x] = src[static_cast<int64_t>(ti + r) * D + tj + x];
  __syncthreads();
#pragma unroll
  for (int r = y; r < 32; r += 8) dst[static_cast<int64_t>(tj + r) * D + ti + x] = f32_to_bf16(tile[x][r]);
}

// G_s = sum of its chunk partials, in chunk order (the order the state pass's partials were
// always added in), for every unit of the window.
template <int D>
__global__ __launch_bounds__(256) void k_gsum(const WindowArgs a) {
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t e4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // float4 index
  if (e4 >= static_cast<int64_t>(a.W) * a.B * a.H * (DD / 4)) return;
  const int64_t u = e4 / (DD / 4), w = 4 * (e4 % (DD / 4));
  f32x4 sum = *reinterpret_cast<const f32x4*>(a.ws.g + u * a.chk * DD + w);
  for (int c = 1; c < a.chk; ++c) sum += *reinterpret_cast<const f32x4*>(a.ws.g + (u * a.chk + c) * DD + w);
  *reinterpret_cast<f32x4*>(a.ws.gs + u * DD + w) = sum;
}

template <int D>
hipError_t launch_chain_d(const WindowArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  if (a.delta) {
    // with several chunks, sum the Gram partials once instead of in every workgroup
    const float* gsum = a.ws.g;
    if (a.chk > 1) {
      const int64_t n4 = static_cast<int64_t>(a.W) * BH * D * D / 4;
      hipLaunchKernelGGL((k_gsum<D>), dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st, a);
      gsum = a.ws.gs;
    }
    const dim3 block(4 * D);
    // 16 rows of M^T per workgroup once that still gives every compute unit a workgroup
    // (one workgroup per compute unit: 152 KB of LDS), else 4
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    const bool wide = BH * (D / 16) >= cus;
    const dim3 grid(BH * (D / (wide ? 16 : 4)));
    auto go = [&](auto chk_c, auto bf_c) {
      constexpr int C = decltype(chk_c)::value;
      constexpr bool BF = decltype(bf_c)::value;
      if (wide) hipLaunchKernelGGL((k_chain_delta<D, C, BF, 4>), grid, block, 0, st, a, gsum);
      else hipLaunchKernelGGL((k_chain_delta<D, C, BF, 1>), grid, block, 0, st, a, gsum);
    };
    if (!a.bf16) go(std::integral_constant<int, 1>{}, std::false_type{});
    else if (a.chk == 1) go(std::integral_constant<int, 1>{}, std::true_type{});
    else if (a.chk == 2) go(std::integral_constant<int, 2>{}, std::true_type{});
    else if (a.chk <= 4) go(std::integral_constant<int, 4>{}, std::true_type{});
    else go(std::integral_constant<int, 8>{}, std::true_type{});
  } else {
    // 8 rows per workgroup (128 threads) while (b,h) pairs x D / 16 leave compute units idle
    auto go = [&](auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      const dim3 grid(BH * (D / RB)), block(16 * RB);
      if (!a.bf16) hipLaunchKernelGGL((k_chain_linear<D, 1, false, RB>), grid, block, 0, st, a);
      else if (a.chk == 1) hipLaunchKernelGGL((k_chain_linear<D, 1, true, RB>), grid, block, 0, st, a);
      else if (a.chk == 2) hipLaunchKernelGGL((k_chain_linear<D, 2, true, RB>), grid, block, 0, st, a);
      else if (a.chk <= 4) hipLaunchKernelGGL((k_chain_linear<D, 4, true, RB>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k_chain_linear<D, 8, true, RB>), grid, block, 0, st, a);
    };
    if (BH * (D / 16) < kChainFillWorkgroups && D >= 64 && 16 * 8 >= D) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain(const WindowArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_chain_d<128>(a, st) : launch_chain_d<64>(a, st);
}

hipError_t launch_state_to_mt(const float* M, void* mt, int pairs, int D, hipStream_t st) {
  const int tb = (D / 32) * (D / 32);
  if (D == 128)
    hipLaunchKernelGGL((k_state_to_mt<128>), dim3(pairs * tb), dim3(256), 0, st, M, static_cast<uint16_t*>(mt));
  else
    hipLaunchKernelGGL((k_state_to_mt<64>), dim3(pairs * tb), dim3(256), 0, st, M, static_cast<uint16_t*>(mt));
  return hipGetLastError();
}

}  // namespace infini
