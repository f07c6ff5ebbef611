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

// Delta rule, G_s summed over the chunks beforehand (k_gsum).  A workgroup owns four
// rows of M^T of one (b,h); thread (r, i) owns row rb + r, column i (the row is the same
// for the whole wave, so the reads of M^T rows are broadcasts; thread i reads row i of
// G_s).  Nothing but M^T itself depends on the chain, so step s + 1's G and U^T / key-sum
// partials are loaded into registers while step s multiplies, and G_{s+1} is staged into
// the other of two LDS buffers at the end of step s.  One barrier per step.  Two waves
// per SIMD, so that one wave's LDS latency is covered by the other's FMAs.  Rows of M^T
// evolve independently, so workgroups never wait on each other.
template <int D, int CHK, bool BF16>
__global__ __launch_bounds__(4 * D, 1) void k_chain_delta(const WindowArgs a, const float* __restrict__ gsum) {
  constexpr int NT = 4 * D;
  constexpr int GP = D + 4;               // LDS row pitch of G and of the M^T rows (floats)
  constexpr int GV = D * D / 4 / NT;      // float4 elements of G_s per thread
  __shared__ __align__(16) float g_lds[2][D][GP];
  __shared__ __align__(16) float m_lds[2][4][GP];

  const int BH = a.B * a.H;
  const int W = a.W;
  const int bh = blockIdx.x / (D / 4);
  const int rb = (blockIdx.x % (D / 4)) * 4;
  const int tid = threadIdx.x;
  const int r = tid / D, i = tid % D;     // r is wave-uniform (D is a multiple of 64)
  const int row = rb + r;                 // this thread's row of M^T
  const int64_t DD = static_cast<int64_t>(D) * D;

  // M^T[row][i] = M[i][row]
  float m = a.zero_state ? 0.f : a.M[bh * DD + static_cast<int64_t>(i) * D + row];
  const bool zown = rb == 0 && tid < D;
  float z = zown && !a.zero_state ? a.z[static_cast<int64_t>(bh) * D + tid] : 0.f;

  // what one step loads ahead of the chain
  struct Pre {
    f32x4 g[GV];
    float up[CHK];
    float dz[CHK];
  };
  auto fetch = [&](int s, Pre& p) __attribute__((always_inline)) {
    const int64_t u = static_cast<int64_t>(min(s, W - 1)) * BH + bh;
    const float* src = gsum + u * DD;
#pragma unroll
    for (int v = 0; v < GV; ++v) p.g[v] = *reinterpret_cast<const f32x4*>(src + 4 * (tid + v * NT));
#pragma unroll
    for (int c = 0; c < CHK; ++c) {
      p.up[c] = a.ws.u[(u * CHK + c) * DD + static_cast<int64_t>(row) * D + i];
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
    const int64_t off = u * DD + static_cast<int64_t>(row) * D + i;
    if constexpr (BF16) static_cast<uint16_t*>(a.ws.mt)[off] = f32_to_bf16(m);
    else static_cast<float*>(a.ws.mt)[off] = m;
    if (zown) {
      a.ws.zb[u * D + tid] = z;
      float dz = 0.f;
#pragma unroll
      for (int c = 0; c < CHK; ++c) dz += p.dz[c];
      z += dz;
    }
    m_lds[b][r][i] = m;
    __syncthreads();   // G_s and this step's rows of M^T are in LDS
    // (M^T G^T)[row][i] = sum_k M^T[row][k] G[i][k], as four interleaved partial sums
    // (k mod 4); k in blocks of 16 whose 8 LDS reads are issued together
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int kk = 0; kk < D; kk += 16) {
      f32x4 gk[4], mk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gk[j] = *reinterpret_cast<const f32x4*>(&g_lds[b][i][kk + 4 * j]);
        mk[j] = *reinterpret_cast<const f32x4*>(&m_lds[b][r][kk + 4 * j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(mk[j][e], gk[j][e], acc[e]);
    }
    float ut = 0.f;
#pragma unroll
    for (int c = 0; c < CHK; ++c) ut += p.up[c];
    m = (m - ((acc[0] + acc[1]) + (acc[2] + acc[3]))) + ut;
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
  a.M[bh * DD + static_cast<int64_t>(i) * D + row] = m;
  if (zown) a.z[static_cast<int64_t>(bh) * D + tid] = z;
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
    const dim3 grid(BH * (D / 4));
    const dim3 block(4 * D);
    if (!a.bf16) hipLaunchKernelGGL((k_chain_delta<D, 1, false>), grid, block, 0, st, a, gsum);
    else if (a.chk == 1) hipLaunchKernelGGL((k_chain_delta<D, 1, true>), grid, block, 0, st, a, gsum);
    else if (a.chk == 2) hipLaunchKernelGGL((k_chain_delta<D, 2, true>), grid, block, 0, st, a, gsum);
    else if (a.chk <= 4) hipLaunchKernelGGL((k_chain_delta<D, 4, true>), grid, block, 0, st, a, gsum);
    else hipLaunchKernelGGL((k_chain_delta<D, 8, true>), grid, block, 0, st, a, gsum);
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
