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
// K and V tiles (64 keys x d, row-major as in memory) are staged in LDS, double buffered,
// prefetched into registers one tile ahead.  The V^T operand of O^T += V^T P^T is read
// with LDS transpose reads, in the key order the S^T result registers hold.  The online softmax is
// in the exp2 domain with the scale folded in, and rescales the accumulator lazily: only
// when a row maximum grows by more than 2^8 (exact: the final division uses the same
// stale maximum).  The gated result is staged through LDS and written once with
// coalesced 16-byte stores.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infini {

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;   // queries per workgroup
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
__global__ __launch_bounds__(kThreads, 2) void k_attn_bf16(const WindowArgs a) {
  constexpr int KP = D + 8;          // K tile row pitch (bf16 elements)
  constexpr int VP = D + 32;         // V tile row pitch: conflict-free transpose reads
  constexpr int KS = D / 16;         // k-steps over the head dimension
  constexpr int DB = D / 32;         // 32-row blocks of the head dimension
  constexpr int KCH = kBN * D / 8 / kThreads;  // 16-byte K (and V) chunks per thread per tile
  constexpr int OP = D + 8;          // output staging row pitch

  __shared__ __align__(16) uint16_t k_lds[2][kBN][KP];
  __shared__ __align__(16) uint16_t v_lds[2][kBN][VP];
  static_assert(sizeof(uint16_t) * 4 * 32 * OP <= sizeof(uint16_t) * 2 * kBN * KP, "staging fits");

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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int qw0 = q0 + 32 * wave;
  const int q = qw0 + l32;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + row0 * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + row0 * D;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + row0 * D;

  // Q as the B operand of S^T: lane holds Q[q][16 ks + 8 hl .. +7]; rows >= n read as 0
  u32x4 qreg[KS];
  {
    const auto qr = buffer_rsrc(qg, static_cast<uint32_t>(n) * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = buffer_ld16(qr, (static_cast<uint32_t>(q) * D + 16 * ks + 8 * hl) * 2);
  }

  // per-thread byte offsets of the K/V chunks inside a tile, and their LDS slots
  uint32_t g_off[KCH];
  int lk_off[KCH], lv_off[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int id = tid + kThreads * i;
    const int row = id / (D / 8), c = id % (D / 8);
    g_off[i] = static_cast<uint32_t>(row * D + 8 * c) * 2;
    lk_off[i] = row * KP + 8 * c;
    lv_off[i] = row * VP + 8 * c;
  }
  const int nkv = (min(q0 + kBM, n) + kBN - 1) / kBN;
  u32x4 kpre[KCH], vpre[KCH];
  auto prefetch = [&](int j) {
    // the resource ends at the segment end: keys past it load as zeros
    const int kv0 = j * kBN;
    const uint32_t bytes = static_cast<uint32_t>(n - kv0) * D * 2;
    const auto kr = buffer_rsrc(kg + static_cast<int64_t>(kv0) * D, bytes);
    const auto vr = buffer_rsrc(vg + static_cast<int64_t>(kv0) * D, bytes);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      kpre[i] = buffer_ld16(kr, g_off[i]);
      vpre[i] = buffer_ld16(vr, g_off[i]);
    }
  };
  auto commit = [&](uint16_t* kb, uint16_t* vb) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      st16(kb + lk_off[i], kpre[i]);
      st16(vb + lv_off[i], vpre[i]);
    }
  };
  // lane offsets of the K operand reads, and of the V^T transpose reads: k-slot (hl, i) of
  // k-step j4 is key 16 j4 + 8 (i / 4) + 4 hl + i % 4, the key the S^T register feeding
  // that slot holds
  const int k_rd = l32 * KP + 8 * hl;
  const int v_rd = (4 * hl + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  prefetch(0);
  commit(&k_lds[0][0][0], &v_lds[0][0][0]);
  __syncthreads();

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;   // running row maximum, scaled (log2 domain)
  float l_part = 0.f;        // this lane's half of the row sum
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = zero16();

  auto step = [&](int j, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* kt = &k_lds[buf][0][0];
    const uint16_t* vt = &v_lds[buf][0][0];
    const bool more = j + 1 < nkv;
    if (more) prefetch(j + 1);
    const int kv0 = j * kBN;
    if (kv0 <= qw0 + 31) {
      // ---- S^T = K Q^T for 64 keys x 32 queries
      f32x16 acc_s[2] = {zero16(), zero16()};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {   // two independent accumulation chains
          const bf16x8 ak = as_bf16x8(ld16(kt + k_rd + 32 * kb * KP + 16 * ks));
          acc_s[kb] = mfma32x32x16(ak, as_bf16x8(qreg[ks]), acc_s[kb]);
        }
      // ---- causal mask on tiles that reach past this wave's first query:
      // register r of block kb holds key kv0 + 32 kb + 8 (r / 4) + 4 hl + r % 4
      if (kv0 + kBN - 1 > qw0) {
        const int lim = q - kv0 - 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) acc_s[kb][r] = -INFINITY;
      }
      // ---- row maximum (this lane's 32 keys, then the other half of the row)
      float mx = acc_s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc_s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * c2;
      if (__any(mxs > m_run + kTau)) {
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      }
      // ---- P = exp2(scale * S - m), row sums, bf16 B operands of O^T
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(acc_s[kb][r], c2, -m_run));
          acc_s[kb][r] = p;
          ls += p;
        }
      l_part += ls;
      bf16x8 pb[4];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x16& sv = acc_s[j4 >> 1];
        const int r0 = 8 * (j4 & 1);
        pb[j4] = as_bf16x8(u32x4{pack_bf16x2(sv[r0 + 0], sv[r0 + 1]), pack_bf16x2(sv[r0 + 2], sv[r0 + 3]),
                                 pack_bf16x2(sv[r0 + 4], sv[r0 + 5]), pack_bf16x2(sv[r0 + 6], sv[r0 + 7])});
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const uint16_t* vp = vt + v_rd + 16 * j4 * VP + 32 * db;
          const u32x2 v0 = lds_read_tr16(vp);
          const u32x2 v1 = lds_read_tr16(vp + 8 * VP);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
          acc_o[db] = mfma32x32x16(av, pb[j4], acc_o[db]);
        }
    }
    if (more) commit(&k_lds[buf ^ 1][0][0], &v_lds[buf ^ 1][0][0]);
    __syncthreads();
  };
  for (int j = 0; j < nkv; j += 2) {
    step(j, IC<0>{});
    if (j + 1 < nkv) step(j + 1, IC<1>{});
  }

  // ---------------------------------------------------------------- epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv_l = 1.f / l_tot;

  // sigma(Q) as the B operand of the retrieval, and the denominator sigma(q) . z_{s-1}
  const float* zb = a.ws.zb + static_cast<int64_t>(u) * D;
  float den = 0.f;
  bf16x8 sq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(zb + 16 * ks + 8 * hl);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(zb + 16 * ks + 8 * hl + 4);
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
  den += __shfl_xor(den, 32);
  const float inv_den = 1.f / (den + a.eps);
  const float g = a.gate_g[h], omg = a.gate_omg[h];

  const uint16_t* mt = static_cast<const uint16_t*>(a.ws.mt) + static_cast<int64_t>(u) * D * D;
  uint16_t(*o_lds)[OP] = reinterpret_cast<uint16_t(*)[OP]>(&k_lds[0][0][0]) + 32 * wave;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 acc_m = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 am = as_bf16x8(ld16(mt + static_cast<int64_t>(32 * db + l32) * D + 16 * ks + 8 * hl));
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
      st8(&o_lds[l32][32 * db + 8 * r4 + 4 * hl],
          u32x2{pack_bf16x2(o[4 * r4], o[4 * r4 + 1]), pack_bf16x2(o[4 * r4 + 2], o[4 * r4 + 3])});
  }
  __syncthreads();
  uint16_t* og = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int i = 0; i < 32 * D / 8 / 64; ++i) {
    const int id = lane + 64 * i;
    const int row = id / (D / 8), c = id % (D / 8);
    if (qw0 + row < n) st16(og + (row0 + qw0 + row) * D + 8 * c, ld16(&o_lds[row][8 * c]));
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
