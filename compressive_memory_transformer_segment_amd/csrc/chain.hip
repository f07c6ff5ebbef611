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
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kThreads = 256;

template <int D, int EPT, int CHK, bool BF16>
__global__ __launch_bounds__(kThreads) void k_chain_linear(const WindowArgs a) {
  constexpr int CG = D / EPT;             // thread columns per row
  constexpr int RB = kThreads / CG;       // rows of M^T per workgroup
  constexpr int kBatch = 8;               // segments whose partials are loaded together
  const int BH = a.B * a.H;
  const int bh = blockIdx.x / (D / RB);
  const int rb = (blockIdx.x % (D / RB)) * RB;
  const int tid = threadIdx.x;
  const int r = tid / CG, cg = tid % CG;
  const int dv = rb + r;
  const int i0 = cg * EPT;
  const int64_t DD = static_cast<int64_t>(D) * D;

  float m[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) m[e] = a.zero_state ? 0.f : a.M[bh * DD + static_cast<int64_t>(i0 + e) * D + dv];
  const bool zown = rb == 0 && tid < D;
  float z = zown && !a.zero_state ? a.z[static_cast<int64_t>(bh) * D + tid] : 0.f;

  for (int s0 = 0; s0 < a.W; s0 += kBatch) {
    // all chunk partials of the batch are independent of the chain: issue them together
    float ut[kBatch][CHK][EPT];
    float dzv[kBatch][CHK];
#pragma unroll
    for (int sb = 0; sb < kBatch; ++sb) {
      const int s = min(s0 + sb, a.W - 1);
      const int64_t u = static_cast<int64_t>(s) * BH + bh;
#pragma unroll
      for (int c = 0; c < CHK; ++c) {
        const int64_t slot = u * CHK + c;
        const float* src = a.ws.u + slot * DD + static_cast<int64_t>(dv) * D + i0;
        if constexpr (EPT == 2) {
          const f32x2 v = *reinterpret_cast<const f32x2*>(src);
          ut[sb][c][0] = v[0];
          ut[sb][c][1] = v[1];
        } else {
#pragma unroll
          for (int e = 0; e < EPT; ++e) ut[sb][c][e] = src[e];
        }
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
        if constexpr (EPT == 2) {
          *reinterpret_cast<uint32_t*>(mt) = pack_bf16x2(m[0], m[1]);
        } else {
#pragma unroll
          for (int e = 0; e < EPT; ++e) mt[e] = f32_to_bf16(m[e]);
        }
      } else {
        float* mt = static_cast<float*>(a.ws.mt) + off;
#pragma unroll
        for (int e = 0; e < EPT; ++e) mt[e] = m[e];
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
        for (int c = 0; c < CHK; ++c) add += ut[sb][c][e];
        m[e] += add;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) a.M[bh * DD + static_cast<int64_t>(i0 + e) * D + dv] = m[e];
  if (zown) a.z[static_cast<int64_t>(bh) * D + tid] = z;
}

// Delta rule: each step needs the workgroup's rows of M^T in full and all of G_s.
// Thread (r, cg) owns row rb + r and columns cg + CG*e (strided, so that lanes read
// consecutive rows of G in LDS).  All loads of a step that do not depend on the chain (the
// U^T, dz and G partials) are issued in batches before they are used.
template <int D, int EPT, int CHK, bool BF16>
__global__ __launch_bounds__(kThreads) void k_chain_delta(const WindowArgs a) {
  constexpr int CG = D / EPT;
  constexpr int RB = kThreads / CG;
  constexpr int GP = D + 4;               // LDS row pitch of G (floats)
  constexpr int MP = D + 4;               // LDS row pitch of the M^T rows
  constexpr int IT = D * D / 4 / kThreads;   // float4 elements of G per thread
  constexpr int NB4 = CHK >= 8 ? 2 : 4;      // float4 elements per load batch
  static_assert(IT % NB4 == 0, "whole batches");
  __shared__ __align__(16) float g_lds[D][GP];
  __shared__ __align__(16) float m_lds[RB][MP];

  const int BH = a.B * a.H;
  const int bh = blockIdx.x / (D / RB);
  const int rb = (blockIdx.x % (D / RB)) * RB;
  const int tid = threadIdx.x;
  const int r = tid / CG, cg = tid % CG;
  const int dv = rb + r;
  const int64_t DD = static_cast<int64_t>(D) * D;

  float m[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) m[e] = a.zero_state ? 0.f : a.M[bh * DD + static_cast<int64_t>(cg + CG * e) * D + dv];
  const bool zown = rb == 0 && tid < D;
  float z = zown && !a.zero_state ? a.z[static_cast<int64_t>(bh) * D + tid] : 0.f;

  for (int s = 0; s < a.W; ++s) {
    const int64_t u = static_cast<int64_t>(s) * BH + bh;
    const int64_t off = u * DD + static_cast<int64_t>(dv) * D;
    // this step's U^T and dz partials
    float up[EPT][CHK];
#pragma unroll
    for (int c = 0; c < CHK; ++c)
#pragma unroll
      for (int e = 0; e < EPT; ++e) up[e][c] = a.ws.u[(u * CHK + c) * DD + static_cast<int64_t>(dv) * D + cg + CG * e];
    float dzp[CHK];
#pragma unroll
    for (int c = 0; c < CHK; ++c) dzp[c] = a.ws.dz[(u * CHK + c) * D + (tid & (D - 1))];   // used by owners only
    // record the state this segment reads
    if constexpr (BF16) {
      uint16_t* mt = static_cast<uint16_t*>(a.ws.mt) + off;
#pragma unroll
      for (int e = 0; e < EPT; ++e) mt[cg + CG * e] = f32_to_bf16(m[e]);
    } else {
      float* mt = static_cast<float*>(a.ws.mt) + off;
#pragma unroll
      for (int e = 0; e < EPT; ++e) mt[cg + CG * e] = m[e];
    }
    if (zown) {
      a.ws.zb[u * D + tid] = z;
      float dz = 0.f;
#pragma unroll
      for (int c = 0; c < CHK; ++c) dz += dzp[c];
      z += dz;
    }
    // stage G_s (sum of the chunk partials, in chunk order) and the rows of M^T
#pragma unroll
    for (int b = 0; b < IT; b += NB4) {
      f32x4 gp[NB4][CHK];
#pragma unroll
      for (int i = 0; i < NB4; ++i) {
        const int e4 = tid + (b + i) * kThreads;
        const int row = (e4 * 4) / D, col = (e4 * 4) % D;
#pragma unroll
        for (int c = 0; c < CHK; ++c)
          gp[i][c] = *reinterpret_cast<const f32x4*>(a.ws.g + (u * CHK + c) * DD + row * D + col);
      }
#pragma unroll
      for (int i = 0; i < NB4; ++i) {
        const int e4 = tid + (b + i) * kThreads;
        const int row = (e4 * 4) / D, col = (e4 * 4) % D;
        f32x4 gs = gp[i][0];
#pragma unroll
        for (int c = 1; c < CHK; ++c) gs += gp[i][c];
        *reinterpret_cast<f32x4*>(&g_lds[row][col]) = gs;
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) m_lds[r][cg + CG * e] = m[e];
    __syncthreads();
    // (M^T G^T)[dv][i] = sum_k M^T[dv][k] G[i][k]
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll 2
    for (int k = 0; k < D; k += 4) {
      const f32x4 mk = *reinterpret_cast<const f32x4*>(&m_lds[r][k]);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const f32x4 gk = *reinterpret_cast<const f32x4*>(&g_lds[cg + CG * e][k]);
        acc[e] += mk[0] * gk[0] + mk[1] * gk[1] + mk[2] * gk[2] + mk[3] * gk[3];
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float ut = 0.f;
#pragma unroll
      for (int c = 0; c < CHK; ++c) ut += up[e][c];
      m[e] = (m[e] - acc[e]) + ut;
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) a.M[bh * DD + static_cast<int64_t>(cg + CG * e) * D + dv] = m[e];
  if (zown) a.z[static_cast<int64_t>(bh) * D + tid] = z;
}

template <int D>
hipError_t launch_chain_d(const WindowArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  if (a.delta) {
    constexpr int EPT = 16 * D / kThreads;        // 16 rows of M^T per workgroup
    const dim3 grid(BH * (D / 16));
    if (!a.bf16) hipLaunchKernelGGL((k_chain_delta<D, EPT, 1, false>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk == 1) hipLaunchKernelGGL((k_chain_delta<D, EPT, 1, true>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk == 2) hipLaunchKernelGGL((k_chain_delta<D, EPT, 2, true>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk <= 4) hipLaunchKernelGGL((k_chain_delta<D, EPT, 4, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_chain_delta<D, EPT, 8, true>), grid, dim3(kThreads), 0, st, a);
  } else {
    constexpr int EPT = 2;
    constexpr int RB = kThreads / (D / EPT);
    const dim3 grid(BH * (D / RB));
    if (!a.bf16) hipLaunchKernelGGL((k_chain_linear<D, EPT, 1, false>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk == 1) hipLaunchKernelGGL((k_chain_linear<D, EPT, 1, true>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk == 2) hipLaunchKernelGGL((k_chain_linear<D, EPT, 2, true>), grid, dim3(kThreads), 0, st, a);
    else if (a.chk <= 4) hipLaunchKernelGGL((k_chain_linear<D, EPT, 4, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_chain_linear<D, EPT, 8, true>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain(const WindowArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_chain_d<128>(a, st) : launch_chain_d<64>(a, st);
}

}  // namespace infini
