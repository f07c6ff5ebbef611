// Backward pass of the Infini-attention layer: gradients of the outputs of a stream with
// respect to Q, K, V, the gate logits and the initial state, back through the whole M / z
// recurrence (backpropagation through time over the segments; "Training Infrastructure
// for Recurrent Attention" in the architecture summary of arXiv 2404.07143), with the
// forward recomputed first (the caller's forward keeps nothing).
//
// Per segment s, with u = sigma(Q), den = u z_{s-1} + eps, g = sigmoid(beta):
//   O = g A_mem + (1 - g) A_dot                                          (Eq. 10)
//   gate:       dbeta += g (1 - g) sum dO . (A_mem - A_dot)
//   local (Eq. 6), with dA_dot = (1 - g) dO and P = exp2(c q.k - lse):
//               dV += (1 - g) P^T dO,  dS = P o (dO V^T - D),  D_t = dO_t . A_dot_t,
//               dQ += (1 - g) scale dS K,  dK += (1 - g) scale dS^T Q
//   retrieval (Eq. 7), dnum = g dO / den, dden_t = -g dO_t . A_mem_t / den_t:
//               dQ += (dnum M_{s-1}^T + dden z_{s-1}^T) o sigma'(Q)
//               dL/dM_{s-1} += u^T dnum,  dL/dz_{s-1} += u^T dden
//   update (Eq. 8 / 9), G_s = dL/dM_s, g_s = dL/dz_s, w = sigma(K):
//     linear:   dV += w G_s,  dw = V G_s^T + g_s,  dL/dM_{s-1} += G_s,  dL/dz_{s-1} += g_s
//     delta:    R = w M_{s-1} / denk, denk = w z_{s-1} + eps, Y = w G_s:
//               dV += Y,  dw = (V - R) G_s^T - (Y / denk) M_{s-1}^T + ddenk z_{s-1}^T + g_s,
//               ddenk_t = Y_t . R_t / denk_t,
//               dL/dM_{s-1} += (I - Gram_s) G_s  (Gram_s = w^T diag(1/denk) w, symmetric),
//               dL/dz_{s-1} += g_s + w^T ddenk
//   dK += dw o sigma'(K).
// The sequential parts are two reverse chains per (batch, head): G over d x d matrices and
// g over d-vectors; everything else runs for all segments at once.  The kernels in this file
// are the plain fp32 SIMT formulation (the f32 I/O path) plus the chains, which both paths
// share; the bf16 path's products run on the matrix cores (attention_bwd.hip), and for the
// linear rule the chains run before the dK, dV kernel, which adds the update's part itself.
#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kBT = 256;
constexpr int kTile = 64;   // tokens per tile

template <bool BF16>
__device__ __forceinline__ float ldv(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// sigma'(x) for sigma = ELU + 1: 1 for x > 0, exp(x) otherwise
__device__ __forceinline__ float dsigma(float x) { return x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e); }

struct Pos {
  int u, s_local, bh, h, n;
  int64_t row0;   // [B,H,T] row of the segment's first token
};

__device__ __forceinline__ Pos pos_of(const WindowArgs& w, int u) {
  Pos p;
  const int BH = w.B * w.H;
  p.u = u;
  p.s_local = u / BH;
  p.bh = u % BH;
  p.h = p.bh % w.H;
  p.n = w.seg_tokens(p.s_local);
  p.row0 = static_cast<int64_t>(p.bh) * w.T + static_cast<int64_t>(w.s0 + p.s_local) * w.N;
  return p;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// M_{s-1}[i][j] from the forward's M^T copy ([d_value][d_key], bf16 or fp32)
template <bool BF16>
__device__ __forceinline__ float m_prev(const WindowArgs& w, int u, int D, int i, int j) {
  const int64_t e = static_cast<int64_t>(u) * D * D + static_cast<int64_t>(j) * D + i;
  return ldv<BF16>(w.ws.mt, e);
}

// ---- per-token scalars and gate partials ---------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBT) void k_bwd_prep(const BackwardArgs b) {
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.pt, tile = static_cast<int>(blockIdx.x) % b.pt;
  const Pos p = pos_of(w, u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float g = w.gate_g[p.h], omg = w.gate_omg[p.h];
  const float* zb = w.ws.zb + static_cast<int64_t>(u) * D;
  for (int i = 0; i < kTile / 4; ++i) {
    const int t = tile * kTile + wave * (kTile / 4) + i;
    if (t >= p.n) break;
    const int64_t row = p.row0 + t;
    float dd = 0.f, em = 0.f, dn = 0.f;
    for (int j = lane; j < D; j += 64) {
      const int64_t e = row * D + j;
      const float o = ldv<BF16>(b.dout, e);
      dd = fmaf(o, w.a_dot[e], dd);
      em = fmaf(o, w.a_mem[e], em);
      dn = fmaf(elu_plus_one(ldv<BF16>(w.q, e)), zb[j], dn);
    }
    dd = wave_sum(dd);
    em = wave_sum(em);
    dn = wave_sum(dn) + w.eps;
    if (lane == 0) {
      b.dd[row] = dd;
      b.den[row] = dn;
      b.dden[row] = -g * em / dn;
      b.bq[row] = (em - dd) * g * omg;
    }
  }
}

// ---- dQ: local attention part (query-parallel) + retrieval part -----------------------
template <int D, bool BF16>
__global__ __launch_bounds__(64 * (D / 32)) void k_bwd_dq(const BackwardArgs b) {
  constexpr int TPR = D / 32;   // threads per query, 32 features each
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  __shared__ float dn_lds[kTile][D];
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.pt, tile = static_cast<int>(blockIdx.x) % b.pt;
  const Pos p = pos_of(w, u);
  const int q0 = tile * kTile;
  if (q0 >= p.n) return;
  const int tid = threadIdx.x, qi = tid / TPR, part = tid % TPR, d0 = 32 * part;
  const int q = q0 + qi;
  const bool live = q < p.n;
  const int64_t row = p.row0 + q;
  const float g = w.gate_g[p.h], omg = w.gate_omg[p.h];
  float qv[32], ov[32], acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    qv[i] = live ? ldv<BF16>(w.q_loc, row * D + d0 + i) : 0.f;
    ov[i] = live ? ldv<BF16>(b.dout, row * D + d0 + i) : 0.f;
    acc[i] = 0.f;
  }
  const float lse = live ? w.lse[row] : 0.f, dd = live ? b.dd[row] : 0.f;
  const float c = w.scale_log2;
  const int kv_end = min(q0 + kTile, p.n);
  for (int t0 = 0; t0 < kv_end; t0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * D; e += blockDim.x) {
      const int t = e / D, d = e % D;
      const bool ok = t0 + t < p.n;
      ks[t][d] = ok ? ldv<BF16>(w.k_loc, (p.row0 + t0 + t) * D + d) : 0.f;
      vs[t][d] = ok ? ldv<BF16>(w.v, (p.row0 + t0 + t) * D + d) : 0.f;
    }
    __syncthreads();
    for (int t = 0; t < KT; ++t) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        s = fmaf(qv[i], ks[t][d0 + i], s);
        dp = fmaf(ov[i], vs[t][d0 + i], dp);
      }
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) {
        s += __shfl_xor(s, off);
        dp += __shfl_xor(dp, off);
      }
      const int kv = t0 + t;
      if (kv > q || kv >= p.n) continue;   // uniform within the query's thread group
      const float pr = __builtin_amdgcn_exp2f(fmaf(s, c, -lse));
      const float ds = pr * (dp - dd);
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] = fmaf(ds, ks[t][d0 + i], acc[i]);
    }
  }
  // retrieval: dnum = g dO / den, du = dnum M^T + dden z
  const float den = live ? b.den[row] : 1.f, dden = live ? b.dden[row] : 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) dn_lds[qi][d0 + i] = g * ov[i] / den;
  __syncthreads();
  const float* zb = w.ws.zb + static_cast<int64_t>(u) * D;
  if (!live) return;
  for (int i = 0; i < 32; ++i) {
    const int di = d0 + i;
    float du = dden * zb[di];
    for (int j = 0; j < D; ++j) du = fmaf(dn_lds[qi][j], m_prev<BF16>(w, u, D, di, j), du);
    const float qr = ldv<BF16>(w.q, row * D + di);   // the PE-free Q of the retrieval
    b.dq[row * D + di] = acc[i] * w.scale * omg + du * dsigma(qr);
  }
}

// ---- dK, dV: local attention part (key-parallel) ---------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(64 * (D / 32)) void k_bwd_dkv(const BackwardArgs b) {
  constexpr int TPR = D / 32;
  constexpr int QT = 32;
  __shared__ float qs[QT][D];
  __shared__ float os[QT][D];
  __shared__ float ls[QT], ds_[QT];
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.pt, tile = static_cast<int>(blockIdx.x) % b.pt;
  const Pos p = pos_of(w, u);
  const int k0 = tile * kTile;
  if (k0 >= p.n) return;
  const int tid = threadIdx.x, ki = tid / TPR, part = tid % TPR, d0 = 32 * part;
  const int key = k0 + ki;
  const bool live = key < p.n;
  const int64_t row = p.row0 + key;
  const float omg = w.gate_omg[p.h];
  float kv[32], vv[32], dk[32], dv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    kv[i] = live ? ldv<BF16>(w.k_loc, row * D + d0 + i) : 0.f;
    vv[i] = live ? ldv<BF16>(w.v, row * D + d0 + i) : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const float c = w.scale_log2;
  for (int t0 = k0; t0 < p.n; t0 += QT) {
    __syncthreads();
    for (int e = tid; e < QT * D; e += blockDim.x) {
      const int t = e / D, d = e % D;
      const bool ok = t0 + t < p.n;
      qs[t][d] = ok ? ldv<BF16>(w.q_loc, (p.row0 + t0 + t) * D + d) : 0.f;
      os[t][d] = ok ? ldv<BF16>(b.dout, (p.row0 + t0 + t) * D + d) : 0.f;
    }
    for (int t = tid; t < QT; t += blockDim.x) {
      const bool ok = t0 + t < p.n;
      ls[t] = ok ? w.lse[p.row0 + t0 + t] : 0.f;
      ds_[t] = ok ? b.dd[p.row0 + t0 + t] : 0.f;
    }
    __syncthreads();
    for (int t = 0; t < QT; ++t) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        s = fmaf(qs[t][d0 + i], kv[i], s);
        dp = fmaf(os[t][d0 + i], vv[i], dp);
      }
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) {
        s += __shfl_xor(s, off);
        dp += __shfl_xor(dp, off);
      }
      const int qr = t0 + t;
      if (qr < key || qr >= p.n) continue;
      const float pr = __builtin_amdgcn_exp2f(fmaf(s, c, -ls[t]));
      const float dsv = pr * (dp - ds_[t]);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        dk[i] = fmaf(dsv, qs[t][d0 + i], dk[i]);
        dv[i] = fmaf(pr, os[t][d0 + i], dv[i]);
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    b.dk[row * D + d0 + i] = dk[i] * w.scale * omg;
    b.dv[row * D + d0 + i] = dv[i] * omg;
  }
}

// ---- R_s = sigma(Q)^T dnum and r_s = sigma(Q)^T dden over one chunk of a segment ------
template <int D, bool BF16>
__global__ __launch_bounds__(kBT) void k_bwd_r(const BackwardArgs b) {
  constexpr int RT = 16;               // tokens per LDS tile
  constexpr int TI = D / 16;           // rows per thread: thread (ti, tj) owns a TI x TI block
  __shared__ float sq[RT][D];
  __shared__ float dn[RT][D];
  __shared__ float dz_[RT];
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.rch, ch = static_cast<int>(blockIdx.x) % b.rch;
  const Pos p = pos_of(w, u);
  const float g = w.gate_g[p.h];
  const int per = (w.N + b.rch - 1) / b.rch;
  const int t_lo = ch * per, t_hi = min(p.n, t_lo + per);
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  float acc[TI][TI], rz[TI];
#pragma unroll
  for (int a = 0; a < TI; ++a) {
    rz[a] = 0.f;
#pragma unroll
    for (int c2 = 0; c2 < TI; ++c2) acc[a][c2] = 0.f;
  }
  for (int t0 = t_lo; t0 < t_hi; t0 += RT) {
    __syncthreads();
    for (int e = tid; e < RT * D; e += kBT) {
      const int t = e / D, d = e % D;
      const bool ok = t0 + t < t_hi;
      const int64_t row = p.row0 + t0 + t;
      sq[t][d] = ok ? elu_plus_one(ldv<BF16>(w.q, row * D + d)) : 0.f;
      dn[t][d] = ok ? g * ldv<BF16>(b.dout, row * D + d) / b.den[row] : 0.f;
    }
    for (int t = tid; t < RT; t += kBT) dz_[t] = (t0 + t < t_hi) ? b.dden[p.row0 + t0 + t] : 0.f;
    __syncthreads();
    for (int t = 0; t < RT; ++t) {
      float a_[TI], c_[TI];
#pragma unroll
      for (int a = 0; a < TI; ++a) {
        a_[a] = sq[t][ti * TI + a];
        c_[a] = dn[t][tj * TI + a];
      }
#pragma unroll
      for (int a = 0; a < TI; ++a) {
        rz[a] = fmaf(a_[a], dz_[t], rz[a]);
#pragma unroll
        for (int c2 = 0; c2 < TI; ++c2) acc[a][c2] = fmaf(a_[a], c_[c2], acc[a][c2]);
      }
    }
  }
  float* rp = b.rpart + (static_cast<int64_t>(u) * b.rch + ch) * D * D;
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int c2 = 0; c2 < TI; ++c2) rp[(ti * TI + a) * D + tj * TI + c2] = acc[a][c2];
  if (tj == 0) {
    float* rzp = b.rzpart + (static_cast<int64_t>(u) * b.rch + ch) * D;
#pragma unroll
    for (int a = 0; a < TI; ++a) rzp[ti * TI + a] = rz[a];
  }
}

// ---- reverse chain of G_s = dL/dM_s over the segments.  Columns of G evolve independently
// under both rules ((I - Gram_s) G acts on each column alone), so one workgroup owns a block
// of kChainCols columns of one (batch, head) and walks the segments backwards.
constexpr int kChainCols = 16;
constexpr int kPreCh = 8;   // z chain: R chunk partials per step kept in registers (segments up to 4096 tokens)
// RCH > 0: the linear rule with exactly RCH chunk partials of R per step (their loads run one
// step ahead); RCH == 0: any rule, any chunk count.
template <int D, int RCH>
__global__ __launch_bounds__(kBT) void k_bwd_chain(const BackwardArgs b) {
  constexpr int TPRW = kBT / D;            // threads per row
  constexpr int CPT = kChainCols / TPRW;   // columns per thread
  __shared__ float gl[D][kChainCols + 1];
  const WindowArgs& w = b.w;
  const int nb = D / kChainCols;
  const int bh = static_cast<int>(blockIdx.x) / nb, BH = w.B * w.H;
  const int cb = (static_cast<int>(blockIdx.x) % nb) * kChainCols;
  const int tid = threadIdx.x, i = tid / TPRW, jl = (tid % TPRW) * CPT, j0 = cb + jl;
  float G[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    G[c] = b.dm_final ? b.dm_final[(static_cast<int64_t>(bh) * D + i) * D + j0 + c] : 0.f;
  if constexpr (RCH > 0) {
    // linear: G_{s-1} = G_s + R_s.  The next step's chunk partials of R are loaded while this
    // step stores, so the loads never wait behind one another.
    static_assert(CPT % 4 == 0, "columns per thread in float4 groups");
    f32x4 nx[RCH][CPT / 4];
    auto fetch = [&](int s) __attribute__((always_inline)) {
      const int64_t u = static_cast<int64_t>(max(s, 0)) * BH + bh;
#pragma unroll
      for (int ch = 0; ch < RCH; ++ch) {
        const float* rp = b.rpart + ((u * RCH + ch) * D + i) * D + j0;
#pragma unroll
        for (int v = 0; v < CPT / 4; ++v) nx[ch][v] = *reinterpret_cast<const f32x4*>(rp + 4 * v);
      }
    };
    fetch(w.W - 1);
    for (int s = w.W - 1; s >= 0; --s) {
      float r[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) r[c] = 0.f;
#pragma unroll
      for (int ch = 0; ch < RCH; ++ch)
#pragma unroll
        for (int c = 0; c < CPT; ++c) r[c] += nx[ch][c / 4][c % 4];
      fetch(s - 1);
      float* gm = b.gm + (static_cast<int64_t>(s) * BH + bh) * D * D;
#pragma unroll
      for (int c = 0; c < CPT; ++c) gm[i * D + j0 + c] = G[c];
#pragma unroll
      for (int c = 0; c < CPT; ++c) G[c] += r[c];
    }
  } else {   // delta rule, or more chunks than the registers hold
  for (int s = w.W - 1; s >= 0; --s) {
    const int u = s * BH + bh;
    float* gm = b.gm + static_cast<int64_t>(u) * D * D;
#pragma unroll
    for (int c = 0; c < CPT; ++c) gm[i * D + j0 + c] = G[c];
    float nG[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) nG[c] = G[c];
    if (w.delta) {   // (I - Gram_s) G, Gram_s = sum of the forward's chunk partials (symmetric)
      __syncthreads();
#pragma unroll
      for (int c = 0; c < CPT; ++c) gl[i][jl + c] = G[c];
      __syncthreads();
      for (int k = 0; k < D; ++k) {
        float gr = 0.f;
        for (int ch = 0; ch < w.chk; ++ch)
          gr += w.ws.g[((static_cast<int64_t>(u) * w.chk + ch) * D + i) * D + k];
#pragma unroll
        for (int c = 0; c < CPT; ++c) nG[c] = fmaf(-gr, gl[k][jl + c], nG[c]);
      }
    }
    for (int ch = 0; ch < b.rch; ++ch) {
      const float* rp = b.rpart + (static_cast<int64_t>(u) * b.rch + ch) * D * D;
#pragma unroll
      for (int c = 0; c < CPT; ++c) nG[c] += rp[i * D + j0 + c];
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) G[c] = nG[c];
  }
  }
  if (b.dm0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) b.dm0[(static_cast<int64_t>(bh) * D + i) * D + j0 + c] = G[c];
  }
}

// ---- memory-update part of dK, dV for a tile of tokens (G_s known) ----------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBT) void k_bwd_update(const BackwardArgs b) {
  constexpr int TT = 16;            // tokens per step: 16 threads per token
  constexpr int OPT = D / 16;       // outputs per thread
  __shared__ float gs[D][D + 1];    // G_s
  __shared__ float ms[D][D + 1];    // M_{s-1} (delta)
  __shared__ float wk[TT][D];       // sigma(k)
  __shared__ float vr[TT][D];       // v - R
  __shared__ float dw[TT][D];       // -Y / denk
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.pt, tile = static_cast<int>(blockIdx.x) % b.pt;
  const Pos p = pos_of(w, u);
  const int tid = threadIdx.x, tk = tid / 16, sub = tid % 16;
  const float* gsrc = b.gm + static_cast<int64_t>(u) * D * D;
  for (int e = tid; e < D * D; e += kBT) gs[e / D][e % D] = gsrc[e];
  if (w.delta)
    for (int e = tid; e < D * D; e += kBT) ms[e / D][e % D] = m_prev<BF16>(w, u, D, e / D, e % D);
  const float* zb = w.ws.zb + static_cast<int64_t>(u) * D;
  float cacc[OPT];
#pragma unroll
  for (int o = 0; o < OPT; ++o) cacc[o] = 0.f;
  const int t_lo = tile * kTile, t_hi = min(p.n, t_lo + kTile);
  for (int t0 = t_lo; t0 < t_hi; t0 += TT) {
    __syncthreads();
    const int t = t0 + tk;
    const bool live = t < t_hi;
    const int64_t row = p.row0 + t;
    for (int o = 0; o < OPT; ++o) {
      const int d = sub + 16 * o;
      wk[tk][d] = live ? elu_plus_one(ldv<BF16>(w.k, row * D + d)) : 0.f;
      vr[tk][d] = live ? ldv<BF16>(w.v, row * D + d) : 0.f;
    }
    __syncthreads();
    // Y_j = sum_i w_i G[i][j] (-> dV), and for the delta rule R_j = sum_i w_i M[i][j] / denk
    float Y[OPT], R[OPT];
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      Y[o] = 0.f;
      R[o] = 0.f;
    }
    for (int i2 = 0; i2 < D; ++i2) {
      const float wi = wk[tk][i2];
#pragma unroll
      for (int o = 0; o < OPT; ++o) {
        Y[o] = fmaf(wi, gs[i2][sub + 16 * o], Y[o]);
        if (w.delta) R[o] = fmaf(wi, ms[i2][sub + 16 * o], R[o]);
      }
    }
    float denk = 1.f, ddk = 0.f;
    if (w.delta) {
      float zs = 0.f;
      for (int o = 0; o < OPT; ++o) zs = fmaf(wk[tk][sub + 16 * o], zb[sub + 16 * o], zs);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) zs += __shfl_xor(zs, off);
      denk = zs + w.eps;
      float yr = 0.f;
#pragma unroll
      for (int o = 0; o < OPT; ++o) {
        R[o] /= denk;
        yr = fmaf(Y[o], R[o], yr);
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) yr += __shfl_xor(yr, off);
      ddk = yr / denk;
    }
    if (live) {
#pragma unroll
      for (int o = 0; o < OPT; ++o) b.dv[row * D + sub + 16 * o] += Y[o];
    }
    __syncthreads();   // every thread is done reading wk / vr for Y, R
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      const int d = sub + 16 * o;
      if (w.delta) {
        vr[tk][d] -= R[o];
        dw[tk][d] = -Y[o] / denk;
        if (live) cacc[o] = fmaf(wk[tk][d], ddk, cacc[o]);   // this thread's share of c_s
      }
    }
    __syncthreads();
    // dw_i = sum_j G[i][j] (v - R)_j (+ delta: sum_j M[i][j] dW_j + ddenk z_i)
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      const int i2 = sub + 16 * o;
      float a = 0.f;
      for (int j = 0; j < D; ++j) {
        a = fmaf(gs[i2][j], vr[tk][j], a);
        if (w.delta) a = fmaf(ms[i2][j], dw[tk][j], a);
      }
      if (w.delta) a = fmaf(ddk, zb[i2], a);
      if (live) {
        const float kr = ldv<BF16>(w.k, row * D + i2);
        b.dk[row * D + i2] += a * dsigma(kr);
      }
    }
  }
  if (w.delta) {   // the tile's c partial: sum the TT token slots' shares through LDS
    __syncthreads();
#pragma unroll
    for (int o = 0; o < OPT; ++o) wk[tk][sub + 16 * o] = cacc[o];
    __syncthreads();
    if (tk == 0) {
      float* cp = b.cpart + (static_cast<int64_t>(u) * b.ct + tile) * D;
#pragma unroll
      for (int o = 0; o < OPT; ++o) {
        float sacc = 0.f;
        for (int t2 = 0; t2 < TT; ++t2) sacc += wk[t2][sub + 16 * o];
        cp[sub + 16 * o] = sacc;
      }
    }
  }
}

// ---- reverse chain of g_s = dL/dz_s (d-vectors), one workgroup per (batch, head) -------
template <int D>
__global__ __launch_bounds__(D) void k_bwd_zchain(const BackwardArgs b) {
  const WindowArgs& w = b.w;
  const int bh = static_cast<int>(blockIdx.x), BH = w.B * w.H, i = threadIdx.x;
  float gz = b.dz_final ? b.dz_final[static_cast<int64_t>(bh) * D + i] : 0.f;
  if (!w.delta && b.rch <= kPreCh) {   // linear: next step's partials loaded one step ahead
    float nx[kPreCh];
    auto fetch = [&](int s) __attribute__((always_inline)) {
      const int64_t u = static_cast<int64_t>(max(s, 0)) * BH + bh;
#pragma unroll
      for (int ch = 0; ch < kPreCh; ++ch) nx[ch] = b.rzpart[(u * b.rch + min(ch, b.rch - 1)) * D + i];
    };
    fetch(w.W - 1);
    for (int s = w.W - 1; s >= 0; --s) {
      float r = 0.f;
#pragma unroll
      for (int ch = 0; ch < kPreCh; ++ch) r += ch < b.rch ? nx[ch] : 0.f;
      fetch(s - 1);
      b.gz[(static_cast<int64_t>(s) * BH + bh) * D + i] = gz;
      gz += r;
    }
    if (b.dz0) b.dz0[static_cast<int64_t>(bh) * D + i] = gz;
    return;
  }
  for (int s = w.W - 1; s >= 0; --s) {
    const int u = s * BH + bh;
    b.gz[static_cast<int64_t>(u) * D + i] = gz;
    for (int ch = 0; ch < b.rch; ++ch) gz += b.rzpart[(static_cast<int64_t>(u) * b.rch + ch) * D + i];
    if (w.delta)
      for (int t = 0; t < b.ct; ++t) gz += b.cpart[(static_cast<int64_t>(u) * b.ct + t) * D + i];
  }
  if (b.dz0) b.dz0[static_cast<int64_t>(bh) * D + i] = gz;
}

// ---- dK += g_s o sigma'(K) (every token of segment s receives dL/dz_s) --------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kBT) void k_bwd_final(const BackwardArgs b) {
  const WindowArgs& w = b.w;
  const int u = static_cast<int>(blockIdx.x) / b.pt, tile = static_cast<int>(blockIdx.x) % b.pt;
  const Pos p = pos_of(w, u);
  const float* gz = b.gz + static_cast<int64_t>(u) * D;
  const int t_lo = tile * kTile, t_hi = min(p.n, t_lo + kTile);
  for (int e = threadIdx.x; e < (t_hi - t_lo) * D; e += kBT) {
    const int t = t_lo + e / D, d = e % D;
    const int64_t x = (p.row0 + t) * D + d;
    b.dk[x] += gz[d] * dsigma(ldv<BF16>(w.k, x));
  }
}

// ---- dbeta: the head's per-token gate terms, summed over batch and tokens ----------------
constexpr int kBetaThreads = 1024;
__global__ __launch_bounds__(kBetaThreads) void k_bwd_dbeta(const BackwardArgs b) {
  const WindowArgs& w = b.w;
  const int h = static_cast<int>(blockIdx.x);
  // eight independent partial sums, so that eight loads per thread are in flight at once
  float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int bb = 0; bb < w.B; ++bb) {
    const float* x = b.bq + (static_cast<int64_t>(bb) * w.H + h) * w.T;
    int64_t t = threadIdx.x;
    for (; t + 7 * kBetaThreads < w.T; t += 8 * kBetaThreads) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = x[t + k * kBetaThreads];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc8[k] += v[k];
    }
    for (; t < w.T; t += kBetaThreads) acc8[0] += x[t];
  }
  float acc = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
  __shared__ float red[kBetaThreads / 64];
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < kBetaThreads / 64; ++i) t += red[i];
    b.dbeta[h] = t;
  }
}

template <int D, bool BF16>
hipError_t launch_all(const BackwardArgs& b, hipStream_t st) {
  const WindowArgs& w = b.w;
  const unsigned tiles = static_cast<unsigned>(w.units() * b.pt);
  const unsigned BH = static_cast<unsigned>(w.B * w.H);
  if constexpr (!BF16)   // (the bf16 forward recomputation writes these terms itself)
    hipLaunchKernelGGL((k_bwd_prep<D, BF16>), dim3(tiles), dim3(kBT), 0, st, b);
  if constexpr (BF16) {
    const hipError_t e = launch_bwd_dq_mfma(b, st);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((k_bwd_dq<D, BF16>), dim3(tiles), dim3(64 * (D / 32)), 0, st, b);
  }
  if (BF16 && !w.delta) {
    // linear: the reverse chains need only the R pass, so they run first and the dK, dV
    // kernel adds the memory-update part (sigma(K) G_s, (V G_s^T + g_s) o sigma'(K)) itself
    hipError_t e = launch_bwd_r_mfma(b, st);
    if (e != hipSuccess) return e;
    const dim3 cgrid(BH * (D / kChainCols));
    if (b.rch == 1) hipLaunchKernelGGL((k_bwd_chain<D, 1>), cgrid, dim3(kBT), 0, st, b);
    else if (b.rch == 2) hipLaunchKernelGGL((k_bwd_chain<D, 2>), cgrid, dim3(kBT), 0, st, b);
    else if (b.rch == 4) hipLaunchKernelGGL((k_bwd_chain<D, 4>), cgrid, dim3(kBT), 0, st, b);
    else if (b.rch == 8) hipLaunchKernelGGL((k_bwd_chain<D, 8>), cgrid, dim3(kBT), 0, st, b);
    else hipLaunchKernelGGL((k_bwd_chain<D, 0>), cgrid, dim3(kBT), 0, st, b);
    hipLaunchKernelGGL((k_bwd_zchain<D>), dim3(BH), dim3(D), 0, st, b);
    e = launch_bwd_gpack(b, st);
    if (e == hipSuccess) e = launch_bwd_dkv_mfma(b, true, st);
    if (e != hipSuccess) return e;
  } else {
    if constexpr (BF16) {
      const hipError_t e = launch_bwd_dkv_mfma(b, false, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL((k_bwd_dkv<D, BF16>), dim3(tiles), dim3(64 * (D / 32)), 0, st, b);
    }
    if constexpr (BF16) {
      const hipError_t e = launch_bwd_r_mfma(b, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL((k_bwd_r<D, BF16>), dim3(static_cast<unsigned>(w.units() * b.rch)), dim3(kBT), 0, st, b);
    }
    hipLaunchKernelGGL((k_bwd_chain<D, 0>), dim3(BH * (D / kChainCols)), dim3(kBT), 0, st, b);
    if constexpr (BF16) {
      const hipError_t e = launch_bwd_update_mfma(b, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL((k_bwd_update<D, BF16>), dim3(tiles), dim3(kBT), 0, st, b);
    }
    hipLaunchKernelGGL((k_bwd_zchain<D>), dim3(BH), dim3(D), 0, st, b);
    hipLaunchKernelGGL((k_bwd_final<D, BF16>), dim3(tiles), dim3(kBT), 0, st, b);
  }
  if (!b.skip_dbeta) hipLaunchKernelGGL(k_bwd_dbeta, dim3(static_cast<unsigned>(w.H)), dim3(kBetaThreads), 0, st, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dbeta(const BackwardArgs& b, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_dbeta, dim3(static_cast<unsigned>(b.w.H)), dim3(kBetaThreads), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& b, hipStream_t st) {
  if (b.w.D == 128) return b.w.bf16 ? launch_all<128, true>(b, st) : launch_all<128, false>(b, st);
  if (b.w.D == 64) return b.w.bf16 ? launch_all<64, true>(b, st) : launch_all<64, false>(b, st);
  return hipErrorInvalidValue;
}

}  // namespace infini
