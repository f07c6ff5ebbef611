// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

// Device workspace for one window of W segments.  A "unit" is one (batch, head) pair on
// one segment: u = s_local * (B*H) + b*H + h.
struct Workspace {
  float* dz;        // [U][CHK][D]    per-chunk key sums  sum_t sigma(k_t)
  float* u;         // [U][CHK][D][D] per-chunk (sigma(K)^T V)^T: [d_value][d_key]
  float* g;         // [U][CHK][D][D] per-chunk sigma(K)^T diag(1/den) sigma(K) (delta): [d_key][d_key]
  float* gs;        // [U][D][D]      the same summed over the chunks (delta, bf16, CHK > 1)
  void* mt;         // [U][D][D]      M_{s-1} transposed ([d_value][d_key]); bf16 or f32
  float* zb;        // [U][D]         z_{s-1}
};

struct WindowArgs {
  const void* q;      // PE-free Q: retrieval (sigma(Q))
  const void* k;      // PE-free K: memory update
  const void* v;
  const void* q_loc;  // Q and K of the local softmax attention (position-embedded, or q / k)
  const void* k_loc;
  void* out;
  float* a_mem;      // optional fp32 [B,H,T,D]
  float* a_dot;      // optional fp32 [B,H,T,D]
  float* lse;        // optional fp32 [B,H,T]: log2 of the softmax row sum, in the scaled
                     // log2 domain (P = exp2(scale log2e q.k - lse)); written with a_mem / a_dot
  // backward recomputation (bf16): with bwd_dout set the attention writes, instead of the
  // output, the per-token terms of the gradient, each [B,H,T] fp32 (and lse)
  const void* bwd_dout;
  float* bwd_dd;     // dO . A_dot
  float* bwd_den;    // sigma(q) z_{s-1} + eps
  float* bwd_dden;   // -g dO . A_mem / den
  float* bwd_bq;     // g (1 - g) dO . (A_mem - A_dot)
  int B, H, D;
  int64_t T;         // tokens in the call
  int N;             // segment length
  int S;             // segments in the call
  int n_last;        // tokens of the call's last segment
  int s0;            // first segment of this window (call-relative)
  int W;             // segments in this window
  int chk;           // chunks per segment in the state pass (partials summed by the chain)
  int ch;            // tokens per chunk (multiple of 64)
  bool delta;
  bool bf16;
  bool zero_state;   // the carried M, z are zero (after a reset): read as 0, not from memory
  float eps;
  float scale_log2;  // softmax scale * log2(e)
  float scale;       // softmax scale
  const float* gate_g;    // [H] sigmoid(beta)
  const float* gate_omg;  // [H] 1 - sigmoid(beta)
  float* M;          // state [B,H,D,D]
  float* z;          // state [B,H,D]
  void* mt_cur;      // optional [B,H,D,D] bf16: the chain writes M^T of the window's final state here
  float* z_cur;      // optional [B,H,D]: ... and the final z
  // Split-key mode of the bf16 attention (one segment, few (batch, head) pairs): the keys
  // of a query tile are split into chunks of split_kc tiles processed by different
  // workgroups; each writes its partial softmax state, and the last to finish merges them
  // (in chunk order) and runs the retrieval, gate and store.  split_kc = 0: off.
  int split_kc;
  int split_items;   // items per (batch, head) pair (this segment)
  int split_slots;   // partial slots per (batch, head) pair: the items of a full segment;
                     // chunk c of query tile qt of pair u uses slot
                     // u * split_slots + (chunks of the query tiles before qt in a full segment) + c
  void* split_acc;   // [slots][512 * D bytes] partial O^T per slot, bf16, in result-register order
  float* split_ml;   // [slots][512][2] partial row maximum and row sum per lane
  int* split_cnt;    // [pairs * tiles] chunks finished per query tile (back to 0 after the merge)
  Workspace ws;

  __host__ __device__ int units() const { return W * B * H; }
  __host__ __device__ int seg_tokens(int s_local) const { return (s0 + s_local == S - 1) ? n_last : N; }
};

// Dense projection C = A W^T (bf16 in and out, fp32 accumulation) over rows grouped in
// nb batches of T rows: A[b][t][k] (k < K), W[n][k] row-major (n < N), C[b][t][n].
// Row and column maps let one kernel read the attention output head-major and write
// Q / K / V head-major:
//   A[b][t][k] at a + b*a_sb + (k / a_dk)*a_sh + t*a_st + k % a_dk        (elements)
//   C[b][t][n] at c[n / c_np] + b*c_sb + ((n % c_np) / c_dh)*c_sh + t*c_st + n % c_dh
// Requirements (checked by the caller): K and a_dk multiples of 32, a_st >= 32;
// N, c_np, c_dh multiples of 8; a, w 16-byte aligned, c 8-byte aligned.
struct GemmArgs {
  const void* a;
  int64_t a_sb, a_sh, a_st;
  int a_dk;
  const void* w;
  void* c[3];
  int64_t c_sb, c_sh, c_st;
  int c_np, c_dh;
  int nb, T, N, K;
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

// One decoding step: one token per (batch, head) inside the current segment.
struct DecodeArgs {
  const void* q;          // [B, H, D] this token (io dtype)
  const void* k;
  const void* v;
  void* out;              // [B, H, D]
  void* kc;               // [B, H, N, D] the segment's cached keys; this token goes to row p
  void* vc;
  const float* M;         // [B, H, D, D] M_{s-1} (f32 path)
  const void* mt;         // [B, H, D, D] M_{s-1}^T in bf16 (bf16 path: the forward's retrieval operand)
  const float* z;         // [B, H, D]    z_{s-1}
  const float* gate_g;    // [H]
  const float* gate_omg;  // [H]
  int B, H, D, N;
  int p;                  // tokens of the segment already cached
  bool bf16;
  bool zero_state;        // M_{s-1}, z_{s-1} are zero (read as 0)
  float scale_log2;
  float eps;
  // Split keys (few (batch, head) pairs): nsplit > 1 workgroups per pair, workgroup c
  // taking keys [c chunk, (c + 1) chunk) of the p + 1; each writes its partial softmax state
  // to sp_part (per pair kDecSlots slots of D + 2 floats: D accumulators, the maximum, the
  // row sum; slot kDecSlots - 1: the retrieval numerator and denominator), counts itself in
  // sp_cnt[pair], and the last to count merges the slots in order and writes the output.
  float* sp_part;
  int* sp_cnt;            // [B, H], zero between launches (the merging workgroup resets it)
  int nsplit;
  int chunk;              // a multiple of 128
};

constexpr int kDecSplitMax = 16;               // key chunks per pair at most
constexpr int kDecSlots = kDecSplitMax + 1;    // partial slots per pair (+ the retrieval)

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// Backward pass over one window holding the whole call (s0 = 0, W = S): the forward has
// run on `w` with a_mem, a_dot and lse written, so w.ws holds M_{s-1}^T (mt), z_{s-1} (zb)
// and, for the delta rule, the Gram partials (g) of every segment.
struct BackwardArgs {
  WindowArgs w;
  const void* dout;      // [B,H,T,D] upstream gradient of the output (io dtype)
  float* dd;             // [B,H,T] sum_j dO_tj A_dot_tj
  float* den;            // [B,H,T] sigma(q_t) z_{s-1} + eps
  float* dden;           // [B,H,T] gradient of the retrieval denominator
  float* dq;             // [B,H,T,D] fp32 outputs
  float* dk;
  float* dv;
  float* rpart;          // [U][rch][D][D] sigma(Q)^T dnum over chunks of the segment
  float* rzpart;         // [U][rch][D]    sigma(Q)^T dden
  float* gm;             // [U][D][D]      dL/dM_s (the state after segment s)
  float* cpart;          // [U][ct][D]     delta: sigma(K)^T ddenk per token tile
  float* gz;             // [U][D]         dL/dz_s
  uint16_t* gpk;         // [U][2][D*D]    bf16 linear: G_s packed for the fused dK, dV epilogue
                         //                (16-row groups; rows i, then rows j)
  float* bq;             // [B,H,T]        per-token gate terms g (1 - g) dO . (A_mem - A_dot)
  const float* dm_final; // optional [B,H,D,D] gradient of the final M
  const float* dz_final; // optional [B,H,D]
  float* dm0;            // optional [B,H,D,D] gradient of the initial M
  float* dz0;            // optional [B,H,D]
  float* dbeta;          // [H]
  bool skip_dbeta;       // leave dbeta to a later launch_bwd_dbeta over the whole call
  int rch;               // token chunks of the R pass per segment
  int pt;                // 64-token tiles per segment (prep, dq, dkv, update, final)
  int ct;                // token tiles per segment of the cpart partials (pt, or 128-token tiles)
};

hipError_t launch_backward(const BackwardArgs& b, hipStream_t st);
hipError_t launch_bwd_dbeta(const BackwardArgs& b, hipStream_t st);   // dbeta over all b.w.T tokens
hipError_t launch_bwd_dq_mfma(const BackwardArgs& b, hipStream_t st);    // bf16: dQ (local + retrieval)
hipError_t launch_bwd_dkv_mfma(const BackwardArgs& b, bool fuse_update, hipStream_t st);   // bf16: dK, dV
                                           // (local; + the linear memory-update part if fuse_update)
hipError_t launch_bwd_gpack(const BackwardArgs& b, hipStream_t st);         // bf16 linear: gm -> gpk
hipError_t launch_bwd_update_mfma(const BackwardArgs& b, hipStream_t st);   // bf16: memory-update part of dK, dV
hipError_t launch_bwd_r_mfma(const BackwardArgs& b, hipStream_t st);        // bf16: sigma(Q)^T dnum, sigma(Q)^T dden

hipError_t launch_key_sums(const WindowArgs& a, hipStream_t st);       // delta only
hipError_t launch_state_pass(const WindowArgs& a, hipStream_t st);     // U (+G), dz (linear), V^T
hipError_t launch_chain(const WindowArgs& a, hipStream_t st);          // M/z recurrence
hipError_t launch_state_to_mt(const float* M, void* mt, int pairs, int D, hipStream_t st);   // M -> bf16 M^T
hipError_t launch_attention(const WindowArgs& a, hipStream_t st);      // local attn + retrieval + gate

}  // namespace infini
