// Host side of the C-ABI declared in include/infini_attn.h: handle, state and workspace
// ownership, argument validation, windowing of long streams, and the per-window launch
// sequence (state pass -> chain -> fused attention/retrieval/gate).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <utility>
#include <vector>

#include "../../include/infini_attn.h"
#include "kernels.hpp"

#define INFINI_EXPORT extern "C" __attribute__((visibility("default")))

// Window workspace of infini_attn_forward_stream_noalloc, for callers that cannot allocate
// device memory: one array per device, held from the library's first use on that device
// until the process ends.  Host code never passes this name to a kernel or a copy: it
// resolves the device address once per device (scratch_resolve) and uses that.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct infini_attn {
  infini_attn_config_t cfg;
  int device;
  int D, N, NP, BH;
  bool bf16, delta;
  float scale;
  int window;          // segments per window
  int part_cap;        // chunk-partial slots per (b,h): >= W_call * chk_call
  float* M;            // [B,H,D,D]
  float* z;            // [B,H,D], stored right after M
  float* gate;         // [2H]: sigmoid(beta), 1 - sigmoid(beta)
  bool state_zero = false;   // M, z are logically zero: reset_state ran, memory not yet written
  void* ws_base;
  size_t ws_bytes;
  void* layer_buf = nullptr;   // forward_layer: Q, K, V, A of one window (bf16)
  size_t layer_bytes = 0;
  void* bwd_buf = nullptr;     // backward: recomputed forward parts and gradient scratch
  size_t bwd_bytes = 0;
  void* dec_cache = nullptr;   // decoding: K then V cache of the open segment, [B,H,N,D] each
  float* dec_split = nullptr;  // decoding with split keys: partial slots, then the pair counters
  size_t dec_split_bytes = 0;
  int dec_p = 0;               // tokens of the open decode segment (0: none open)
  // bf16 handles: copies of the carried state for the kernels that read it while a chain
  // may be writing the next one -- M^T in bf16 ([B,H,d_value,d_key], the retrieval operand
  // of one-segment calls and of decoding) and z -- in two buffers: buffer `cur` holds the
  // current state; every chain launch writes the other one and flips `cur` (set_state
  // rebuilds the current one; while state_zero is set the kernels read zeros instead)
  void* mt_buf = nullptr;      // [2][B,H,D,D] bf16
  float* zc_buf = nullptr;     // [2][B,H,D]
  int cur = 0;
  // one-segment calls with few (batch, head) pairs: split-key attention partials and counts,
  // and a second stream on which the memory-update kernels run next to the attention
  void* split_buf = nullptr;
  size_t split_bytes = 0;
  void* split_acc = nullptr;
  float* split_ml = nullptr;
  int* split_cnt = nullptr;
  int split_kc = 0;            // key tiles per chunk
  int split_slots = 0;         // partial slots per (batch, head) pair
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_sp = nullptr, ev_chain = nullptr;
  bool side_pending = false;   // a chain on the side stream may still run (see join_side)
  infini::Workspace ws;
  // per-kernel event timing (measurement only)
  bool profiling = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<std::pair<int, size_t>> ev_marks;   // (kernel kind, index of the start event)
};

namespace {

// Zero fill by a kernel rather than hipMemsetAsync, so that a caller may capture the
// reset in a HIP graph.
__global__ void k_zero_f32(float* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      *reinterpret_cast<float4*>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      for (int64_t k = i; k < n; ++k) p[k] = 0.f;
    }
  }
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + 1023) / 1024, 1024);
  hipLaunchKernelGGL(k_zero_f32, dim3(static_cast<unsigned>(std::max<int64_t>(blocks, 1))), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

std::mutex g_live_mu;
std::unordered_set<const infini_attn*> g_live;

bool live(const infini_attn* h) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return h && g_live.count(h);
}

constexpr size_t kDefaultWorkspaceBudget = size_t(512) << 20;   // bytes
constexpr int kMaxWindow = 64;
// Workgroups the bf16 state pass aims for (segments x chunks): one warp-specialised
// workgroup per compute unit.
constexpr int kStateTargetWorkgroups = 256;

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = prev == dev || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// One chunk-partial slot: key sums, (sigma(K)^T V)^T and, for the delta rule, the Gram term.
size_t part_bytes(const infini_attn& h) {
  const size_t D = h.D, DD = D * D;
  return D * 4 + DD * 4 + (h.delta ? DD * 4 : 0);
}

// Bytes of workspace one window needs, per (b,h) pair, excluding the chunk partials.
size_t unit_bytes(const infini_attn& h) {
  const size_t D = h.D, DD = D * D;
  size_t b = 0;
  b += DD * (h.bf16 ? 2 : 4);        // mt
  b += D * 4;                        // zb
  if (h.delta) b += DD * 4;          // gs
  return b + part_bytes(h);          // at least one chunk slot per unit
}
// Decoding with fewer (batch, head) pairs than this splits the keys so that about this many
// workgroups run, in chunks of at least kDecChunk keys (measured at 8 heads, d = 128,
// N = 2048: batch 1 12.3 against 16.5 us per token, batch 8 15.7 against 17.1; a target of
// 512 workgroups or 128-key chunks made batch 8 slower than no split, the merge's round
// trips costing more than the shorter key streams saved).
constexpr int kDecTargetWorkgroups = 128;
constexpr int kDecChunk = 256;

int chunks_for(const infini_attn& h, int w_call, int part_cap) {
  if (!h.bf16) return 1;
  const int units = w_call * h.BH;
  // a power of two (the chain kernel is specialised on it), at most 8, and no more chunks
  // than 64-token sub-tiles
  const int want = (kStateTargetWorkgroups + units - 1) / units;
  int chk = 1;
  while (chk * 2 <= want && chk * 2 <= 8 && chk * 2 <= std::max(1, h.NP / 64) && w_call * chk * 2 <= part_cap)
    chk *= 2;
  return chk;
}

int chunks_for(const infini_attn& h, int w_call) { return chunks_for(h, w_call, h.part_cap); }

// Chunk-partial slots per (b,h) that windows of up to w segments need.
int part_cap_for(const infini_attn& h, int w) {
  int cap = w;
  if (h.bf16)
    for (int wc = 1; wc <= w; ++wc) cap = std::max(cap, wc * chunks_for(h, wc, 1 << 30));
  return cap;
}

// Workspace layout: one window of units plus the chunk-partial slots.
template <typename F>
void layout(const infini_attn& h, int window, int part_cap, F&& take) {
  const size_t U = size_t(window) * h.BH;
  const size_t P = size_t(part_cap) * h.BH;
  const size_t D = h.D, DD = D * D;
  take(0, P * D * 4);                                // dz
  take(1, P * DD * 4);                               // u
  take(2, h.delta ? P * DD * 4 : 0);                 // g
  take(3, h.delta ? U * DD * 4 : 0);                 // gs
  take(4, U * DD * (h.bf16 ? 2 : 4));                // mt
  take(5, U * D * 4);                                // zb
}

size_t layout_bytes(const infini_attn& h, int window, int part_cap) {
  size_t b = 0;
  layout(h, window, part_cap, [&](int, size_t bytes) { b += align_up(bytes, 256); });
  return b;
}

// The window workspace carved from `base` (256-byte aligned); returns its size in bytes.
size_t carve(const infini_attn& h, int window, int part_cap, void* base, infini::Workspace& ws) {
  char* p = static_cast<char*>(base);
  void* ptrs[6] = {};
  layout(h, window, part_cap, [&](int i, size_t bytes) {
    ptrs[i] = bytes ? p : nullptr;
    p += align_up(bytes, 256);
  });
  ws.dz = static_cast<float*>(ptrs[0]);
  ws.u = static_cast<float*>(ptrs[1]);
  ws.g = static_cast<float*>(ptrs[2]);
  ws.gs = static_cast<float*>(ptrs[3]);
  ws.mt = ptrs[4];
  ws.zb = static_cast<float*>(ptrs[5]);
  return static_cast<size_t>(p - static_cast<char*>(base));
}

// Where a forward call's window workspace lives: segments per window, chunk-partial slots
// per (b,h) and the carved buffers.
struct WindowPlan {
  infini::Workspace ws;
  int window;
  int part_cap;
};

WindowPlan handle_plan(const infini_attn& h) { return WindowPlan{h.ws, h.window, h.part_cap}; }

// Device address of `scratch` on each device (nullptr: not resolved yet).
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;

// Resolves the address of `scratch` on `device`, which must be the current device.
hipError_t scratch_resolve(int device) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (device < 0) return hipErrorInvalidDevice;
  if (static_cast<int>(g_scratch_ptr.size()) <= device) g_scratch_ptr.resize(size_t(device) + 1, nullptr);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return e != hipSuccess ? e : hipErrorInvalidSymbol;
  }
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return device >= 0 && device < static_cast<int>(g_scratch_ptr.size()) ? g_scratch_ptr[device] : nullptr;
}

// The window workspace of one call of S segments carved from the scratch array at
// `base`: the longest window (at most the handle's) whose workspace fits kScratchBytes,
// with chunk-partial slots for exactly the windows the call runs (full ones and the
// last), each chunked as forward_stream chunks a window of its length.
int scratch_plan(const infini_attn& h, int64_t S, void* base, WindowPlan& plan) {
  for (int w = static_cast<int>(std::min<int64_t>(h.window, S)); w >= 1; --w) {
    const int w_last = static_cast<int>(S - (S - 1) / w * w);
    const int cap = h.bf16 ? std::max(w * chunks_for(h, w, 1 << 30), w_last * chunks_for(h, w_last, 1 << 30)) : w;
    if (layout_bytes(h, w, cap) > kScratchBytes) continue;
    plan.window = w;
    plan.part_cap = cap;
    carve(h, w, cap, base, plan.ws);
    return INFINI_OK;
  }
  return INFINI_ERR_SCRATCH;
}

void gate_values(const float* beta, int H, float* out) {
  for (int i = 0; i < H; ++i) {
    const double b = beta[i];
    double g, omg;
    if (std::isnan(b)) {
      g = omg = b;
    } else if (b >= 0) {
      const double e = std::exp(-b);
      g = 1.0 / (1.0 + e);
      omg = e / (1.0 + e);
    } else {
      const double e = std::exp(b);
      g = e / (1.0 + e);
      omg = 1.0 / (1.0 + e);
    }
    out[i] = static_cast<float>(g);
    out[H + i] = static_cast<float>(omg);
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_io(const infini_attn* h, const void* q, const void* k, const void* v, const void* out,
             int64_t n_tokens) {
  if (!q || !k || !v || !out) return INFINI_ERR_INVALID_ARG;
  if (n_tokens < 1) return INFINI_ERR_INVALID_ARG;
  const size_t esz = h->bf16 ? 2 : 4;
  const size_t align = h->bf16 ? 16 : 4;
  for (const void* p : {q, k, v, out})
    if (reinterpret_cast<uintptr_t>(p) % align) return INFINI_ERR_INVALID_ARG;
  const double elems = double(h->BH) * double(n_tokens) * double(h->D);
  if (elems * esz > 9.0e18) return INFINI_ERR_INVALID_ARG;
  const size_t bytes = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * esz;
  for (const void* p : {q, k, v})
    if (overlaps(out, bytes, p, bytes)) return INFINI_ERR_INVALID_ARG;
  return INFINI_OK;
}

// Launch one kernel, bracketed by events when profiling is on.
template <typename F>
hipError_t timed(infini_attn* h, int kind, hipStream_t st, F&& launch) {
  if (!h->profiling) return launch();
  while (h->ev_pool.size() < h->ev_used + 2) {
    hipEvent_t e;
    // timing only: no system-scope fence (cache writeback and invalidate) when the event
    // is recorded, which would otherwise add to the bracketed kernel's time
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) return err;
    h->ev_pool.push_back(e);
  }
  const size_t i = h->ev_used;
  hipError_t e = hipEventRecord(h->ev_pool[i], st);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(h->ev_pool[i + 1], st);
  if (e == hipSuccess) {
    h->ev_marks.emplace_back(kind, i);
    h->ev_used += 2;
  }
  return e;
}

void* mt_of(const infini_attn* h, int i) {
  return h->mt_buf ? static_cast<char*>(h->mt_buf) + size_t(i) * h->BH * h->D * h->D * 2 : nullptr;
}
float* zc_of(const infini_attn* h, int i) {
  return h->zc_buf ? h->zc_buf + size_t(i) * h->BH * h->D : nullptr;
}

// Where the chain of the launch being set up writes its copies of the final state; the
// caller flips h->cur once the chain is enqueued.
void chain_outputs(const infini_attn* h, infini::WindowArgs& a) {
  a.mt_cur = mt_of(h, h->cur ^ 1);
  a.z_cur = zc_of(h, h->cur ^ 1);
}

// Orders stream st after a chain that a one-segment call left running on the side stream
// (every call that reads or writes the state, the workspace or the copies does this first).
hipError_t join_side(infini_attn* h, hipStream_t st) {
  if (!h->side_pending) return hipSuccess;
  const hipError_t e = hipStreamWaitEvent(st, h->ev_chain, 0);
  if (e == hipSuccess) h->side_pending = false;
  return e;
}

int device_compute_units(int device) {
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || c <= 0) {
    (void)hipGetLastError();
    c = 256;
  }
  return c;
}

constexpr int kQueryTile = 256;   // queries per attention item (bf16)
constexpr int kKeyTile = 64;      // keys per attention tile (bf16)

// Split-key chunks of query tile qt of an n-token segment, kc key tiles per chunk.
int split_chunks(int qt, int n, int kc) {
  const int nkv = (std::min(qt * kQueryTile + kQueryTile, n) + kKeyTile - 1) / kKeyTile;
  return (nkv + kc - 1) / kc;
}

// Split-key items of one (batch, head) pair for an n-token segment.
int split_items(int n, int kc) {
  int p = 0;
  for (int qt = 0; qt * kQueryTile < n; ++qt) p += split_chunks(qt, n, kc);
  return p;
}

int run_stream(infini_attn* h, const void* q, const void* k, const void* v, void* out, float* a_mem,
               float* a_dot, int64_t n_tokens, void* hip_stream, const void* q_loc = nullptr,
               const void* k_loc = nullptr, const WindowPlan* plan_in = nullptr) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (h->dec_p > 0) return INFINI_ERR_INVALID_ARG;   // a decode segment is open: flush it first
  int rc = check_io(h, q, k, v, out, n_tokens);
  if (rc) return rc;
  if (!q_loc) q_loc = q;
  if (!k_loc) k_loc = k;
  rc = check_io(h, q_loc, k_loc, v, out, n_tokens);
  if (rc) return rc;
  const size_t part_bytes_out = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * 4;
  for (const float* p : {a_mem, a_dot}) {
    if (!p) continue;
    if (reinterpret_cast<uintptr_t>(p) % 4) return INFINI_ERR_INVALID_ARG;
    if (overlaps(p, part_bytes_out, out, part_bytes_out / (h->bf16 ? 2 : 1))) return INFINI_ERR_INVALID_ARG;
  }
  if (a_mem && a_dot && overlaps(a_mem, part_bytes_out, a_dot, part_bytes_out)) return INFINI_ERR_INVALID_ARG;
  const int64_t S64 = (n_tokens + h->N - 1) / h->N;
  if (S64 > (int64_t(1) << 30)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const WindowPlan plan = plan_in ? *plan_in : handle_plan(*h);

  infini::WindowArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_loc = q_loc;
  a.k_loc = k_loc;
  a.out = out;
  a.a_mem = a_mem;
  a.a_dot = a_dot;
  a.B = h->cfg.batch;
  a.H = h->cfg.heads;
  a.D = h->D;
  a.T = n_tokens;
  a.N = h->N;
  a.S = static_cast<int>(S64);
  a.n_last = static_cast<int>(n_tokens - (S64 - 1) * h->N);
  a.delta = h->delta;
  a.bf16 = h->bf16;
  a.eps = h->cfg.eps;
  a.scale = h->scale;
  a.scale_log2 = static_cast<float>(double(h->scale) * 1.4426950408889634);
  a.gate_g = h->gate;
  a.gate_omg = h->gate + h->cfg.heads;
  a.M = h->M;
  a.z = h->z;
  a.ws = plan.ws;
  a.zero_state = h->state_zero;
  if (join_side(h, st) != hipSuccess) return INFINI_ERR_HIP;
  if (h->split_buf && !plan_in && a.S == 1 && !a_mem && !a_dot) {
    // One segment with few (batch, head) pairs.  The attention reads the carried state
    // (the current bf16 M^T and z copies) and does not depend on this segment's memory
    // update, so the update kernels -- state pass, then the chain, which writes the new
    // state and its copies into the other buffer -- run on the second stream meanwhile.
    // The launch stream waits for the state pass (the last reader of the caller's K, V)
    // before the call's work on it ends; the chain, which touches library memory only, is
    // joined by the next call that needs the state.  The attention splits the keys of a
    // query tile over several workgroups, so that the few pairs fill the compute units.
    a.s0 = 0;
    a.W = 1;
    a.chk = chunks_for(*h, 1, plan.part_cap);
    a.ch = static_cast<int>(align_up(size_t((h->N + a.chk - 1) / a.chk), 64));
    chain_outputs(h, a);
    infini::WindowArgs at = a;
    at.ws.mt = mt_of(h, h->cur);
    at.ws.zb = zc_of(h, h->cur);
    at.split_kc = h->split_kc;
    at.split_items = split_items(a.n_last, h->split_kc);
    at.split_slots = h->split_slots;
    at.split_acc = h->split_acc;
    at.split_ml = h->split_ml;
    at.split_cnt = h->split_cnt;
    hipError_t e = hipEventRecord(h->ev_fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->ev_fork, 0);
    if (e == hipSuccess && h->delta) e = timed(h, 0, h->side, [&] { return infini::launch_key_sums(a, h->side); });
    if (e == hipSuccess) e = timed(h, 1, h->side, [&] { return infini::launch_state_pass(a, h->side); });
    if (e == hipSuccess) e = hipEventRecord(h->ev_sp, h->side);
    if (e == hipSuccess) e = timed(h, 2, h->side, [&] { return infini::launch_chain(a, h->side); });
    if (e == hipSuccess) e = hipEventRecord(h->ev_chain, h->side);
    if (e == hipSuccess) {
      h->side_pending = true;
      h->cur ^= 1;
      h->state_zero = false;
    }
    if (e == hipSuccess) e = timed(h, 3, st, [&] { return infini::launch_attention(at, st); });
    if (e == hipSuccess) e = hipStreamWaitEvent(st, h->ev_sp, 0);
    return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
  }
  for (int s0 = 0; s0 < a.S; s0 += plan.window) {
    a.s0 = s0;
    a.W = std::min(plan.window, a.S - s0);
    a.chk = chunks_for(*h, a.W, plan.part_cap);
    a.ch = static_cast<int>(align_up(size_t((h->N + a.chk - 1) / a.chk), 64));   // trailing chunks may be empty
    hipError_t e = hipSuccess;
    if (h->delta) e = timed(h, 0, st, [&] { return infini::launch_key_sums(a, st); });
    if (e == hipSuccess) e = timed(h, 1, st, [&] { return infini::launch_state_pass(a, st); });
    chain_outputs(h, a);
    if (e == hipSuccess) e = timed(h, 2, st, [&] { return infini::launch_chain(a, st); });
    if (e == hipSuccess) {   // the chain has written the carried state
      h->cur ^= 1;
      h->state_zero = false;
      a.zero_state = false;
    }
    if (e == hipSuccess) e = timed(h, 3, st, [&] { return infini::launch_attention(a, st); });
    if (e != hipSuccess) return INFINI_ERR_HIP;
  }
  return INFINI_OK;
}

// ---- projections (Eq. 5, Eq. 11) -------------------------------------------------------

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Shared argument checks of the projection calls.
int check_layer(const infini_attn* h, int64_t n_tokens, int32_t d_model) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (!h->bf16) return INFINI_ERR_UNSUPPORTED;
  if (n_tokens < 1 || n_tokens > (int64_t(1) << 31) - 1) return INFINI_ERR_INVALID_ARG;
  if (d_model < 32 || d_model % 32 != 0 || d_model > (1 << 16)) return INFINI_ERR_INVALID_ARG;
  return INFINI_OK;
}

// Q/K/V of tokens [t0, t0 + tc) of a stream of T tokens: x [B, T, dm] -> q, k, v
// [B, H, tc, d].
hipError_t launch_qkv(const infini_attn* h, const void* x, int64_t T, int64_t t0, int tc, int dm,
                      const void* w_qkv, void* q, void* k, void* v, hipStream_t st) {
  const int H = h->cfg.heads, D = h->D;
  infini::GemmArgs g{};
  g.a = static_cast<const uint16_t*>(x) + t0 * dm;
  g.a_sb = T * dm;
  g.a_sh = 0;
  g.a_st = dm;
  g.a_dk = dm;
  g.w = w_qkv;
  g.c[0] = q;
  g.c[1] = k;
  g.c[2] = v;
  g.c_np = H * D;
  g.c_dh = D;
  g.c_sh = int64_t(tc) * D;
  g.c_st = D;
  g.c_sb = int64_t(H) * tc * D;
  g.nb = h->cfg.batch;
  g.T = tc;
  g.N = 3 * H * D;
  g.K = dm;
  return infini::launch_gemm(g, st);
}

// O rows [t0, t0 + tc) of a stream of T tokens from A [B, H, tc, d]: out [B, T, dm].
hipError_t launch_out(const infini_attn* h, const void* a, const void* w_o, void* out, int64_t T,
                      int64_t t0, int tc, int dm, hipStream_t st) {
  const int H = h->cfg.heads, D = h->D;
  infini::GemmArgs g{};
  g.a = a;
  g.a_sb = int64_t(H) * tc * D;
  g.a_sh = int64_t(tc) * D;
  g.a_st = D;
  g.a_dk = D;
  g.w = w_o;
  g.c[0] = static_cast<uint16_t*>(out) + t0 * dm;
  g.c[1] = g.c[0];
  g.c[2] = g.c[0];
  g.c_np = dm;
  g.c_dh = dm;
  g.c_sh = 0;
  g.c_st = dm;
  g.c_sb = T * dm;
  g.nb = h->cfg.batch;
  g.T = tc;
  g.N = dm;
  g.K = H * D;
  return infini::launch_gemm(g, st);
}

}  // namespace

INFINI_EXPORT const char* infini_attn_status_string(int status) {
  switch (status) {
    case INFINI_OK: return "ok";
    case INFINI_ERR_INVALID_ARG: return "invalid argument";
    case INFINI_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFINI_ERR_HIP: return "HIP runtime error";
    case INFINI_ERR_OOM: return "out of device memory";
    case INFINI_ERR_SCRATCH: return "one segment's workspace exceeds the static scratch of the allocation-free call";
    default: return "unknown status";
  }
}

INFINI_EXPORT int infini_attn_create(const infini_attn_config_t* cfg, const float* beta_host,
                                     void* hip_stream, infini_attn_t* out) {
  if (!cfg || !beta_host || !out) return INFINI_ERR_INVALID_ARG;
  *out = nullptr;
  const infini_attn_config_t c = *cfg;
  if (c.batch < 1 || c.heads < 1 || c.segment_len < 1) return INFINI_ERR_INVALID_ARG;
  if (c.update != INFINI_UPDATE_LINEAR && c.update != INFINI_UPDATE_DELTA) return INFINI_ERR_INVALID_ARG;
  if (c.io_dtype != INFINI_DTYPE_BF16 && c.io_dtype != INFINI_DTYPE_F32) return INFINI_ERR_INVALID_ARG;
  if (!(c.eps >= 0.f) || !std::isfinite(c.eps)) return INFINI_ERR_INVALID_ARG;
  if (std::isnan(c.softmax_scale) || std::isinf(c.softmax_scale)) return INFINI_ERR_INVALID_ARG;
  if (c.head_dim != 64 && c.head_dim != 128) return INFINI_ERR_UNSUPPORTED;
  if (int64_t(c.batch) * c.heads > (int64_t(1) << 20) || c.segment_len > (1 << 22)) return INFINI_ERR_UNSUPPORTED;

  infini_attn* h = new (std::nothrow) infini_attn{};
  if (!h) return INFINI_ERR_OOM;
  h->cfg = c;
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return INFINI_ERR_HIP; }
  h->D = c.head_dim;
  h->N = c.segment_len;
  h->NP = static_cast<int>(align_up(size_t(c.segment_len), 64));
  h->BH = c.batch * c.heads;
  h->bf16 = c.io_dtype == INFINI_DTYPE_BF16;
  h->delta = c.update == INFINI_UPDATE_DELTA;
  h->scale = c.softmax_scale > 0.f ? c.softmax_scale : static_cast<float>(1.0 / std::sqrt(double(c.head_dim)));

  // window: as many segments as fit the workspace budget (at least one)
  size_t budget = kDefaultWorkspaceBudget;
  if (const char* env = std::getenv("INFINI_ATTN_WORKSPACE_MB")) {
    const long mb = std::strtol(env, nullptr, 10);
    if (mb > 0) budget = size_t(mb) << 20;
  }
  const size_t per_seg = unit_bytes(*h) * h->BH;
  int w = static_cast<int>(std::max<size_t>(1, budget / std::max<size_t>(per_seg, 1)));
  w = std::min(w, kMaxWindow);
  if (c.max_window_segments > 0) w = std::min(w, c.max_window_segments);
  h->window = w;
  // chunk partials: enough slots for the chunking chosen at any window size
  h->part_cap = part_cap_for(*h, w);

  DeviceGuard dg(h->device);
  const size_t DD = size_t(h->D) * h->D;
  const size_t m_bytes = size_t(h->BH) * DD * 4, z_bytes = size_t(h->BH) * h->D * 4;
  const size_t ws_bytes = layout_bytes(*h, h->window, h->part_cap);
  // M and z in one allocation (z follows M), so one fill resets both
  if (hipMalloc(&h->M, m_bytes + z_bytes) != hipSuccess) { (void)hipGetLastError(); delete h; return INFINI_ERR_OOM; }
  h->z = h->M + size_t(h->BH) * DD;
  if (hipMalloc(&h->gate, size_t(2) * c.heads * 4) != hipSuccess ||
      hipMalloc(&h->ws_base, ws_bytes) != hipSuccess) {
    (void)hipFree(h->M); (void)hipFree(h->gate);
    delete h;
    (void)hipGetLastError();
    return INFINI_ERR_OOM;
  }
  h->ws_bytes = carve(*h, h->window, h->part_cap, h->ws_base, h->ws);
  (void)scratch_resolve(h->device);   // for forward_stream_noalloc; checked again there
  if (h->bf16) {
    const size_t mt_bytes = 2 * size_t(h->BH) * DD * 2;
    bool ok = hipMalloc(&h->mt_buf, mt_bytes) == hipSuccess &&
              hipMalloc(reinterpret_cast<void**>(&h->zc_buf), 2 * size_t(h->BH) * h->D * 4) == hipSuccess;
    // split-key attention for one-segment calls when the pairs' query tiles fill at most
    // the compute units: chunks of kc key tiles (a multiple of 4, at most 8 per query tile),
    // the shortest of 8, 12, 16, ... whose items all fit in one round over the compute units
    // (8 heads: kc = 8, 160 items; 32 heads: one chunk per query tile, which measured 11%
    // faster per segment than kc = 8 with 640 items); INFINI_ATTN_SPLIT_KC overrides kc
    const int nq = (h->N + kQueryTile - 1) / kQueryTile;
    const int cus = device_compute_units(h->device);
    if (ok && int64_t(h->BH) * nq <= cus) {
      int kc = 8;
      while (kc < 4 * nq && int64_t(h->BH) * split_items(h->N, std::max(kc, (nq + 7) / 8 * 4)) > cus) kc += 4;
      if (const char* env = std::getenv("INFINI_ATTN_SPLIT_KC")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v >= 4 && v % 4 == 0 && v <= 4096) kc = static_cast<int>(v);
      }
      h->split_kc = std::max(kc, (nq + 7) / 8 * 4);   // 4 nq key tiles in at most 8 chunks
      h->split_slots = split_items(h->N, h->split_kc);
      const size_t slots = size_t(h->BH) * h->split_slots;
      const size_t acc_b = align_up(slots * 512 * h->D, 256), ml_b = align_up(slots * 1024 * 4, 256);
      const size_t cnt_b = align_up(size_t(h->BH) * nq * 4, 256);
      h->split_bytes = acc_b + ml_b + cnt_b;
      ok = hipMalloc(&h->split_buf, h->split_bytes) == hipSuccess &&
           hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&h->ev_sp, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&h->ev_chain, hipEventDisableTiming) == hipSuccess;
      if (ok) {
        h->split_acc = h->split_buf;
        h->split_ml = reinterpret_cast<float*>(static_cast<char*>(h->split_buf) + acc_b);
        h->split_cnt = reinterpret_cast<int*>(static_cast<char*>(h->split_buf) + acc_b + ml_b);
      }
    }
    if (!ok) {
      (void)hipGetLastError();
      {
        std::lock_guard<std::mutex> lk(g_live_mu);
        g_live.insert(h);
      }
      infini_attn_destroy(h);
      return INFINI_ERR_OOM;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(h);
  }
  float* gv = new (std::nothrow) float[2 * c.heads];
  if (!gv) { infini_attn_destroy(h); return INFINI_ERR_OOM; }
  gate_values(beta_host, c.heads, gv);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipMemcpy(h->gate, gv, size_t(2) * c.heads * 4, hipMemcpyHostToDevice);
  delete[] gv;
  if (e == hipSuccess) e = hipMemsetAsync(h->M, 0, m_bytes + z_bytes, st);
  if (e == hipSuccess && h->mt_buf) e = hipMemsetAsync(h->mt_buf, 0, 2 * size_t(h->BH) * DD * 2, st);
  if (e == hipSuccess && h->zc_buf) e = hipMemsetAsync(h->zc_buf, 0, 2 * size_t(h->BH) * h->D * 4, st);
  if (e == hipSuccess && h->split_cnt)
    e = hipMemsetAsync(h->split_cnt, 0, size_t(h->BH) * ((h->N + kQueryTile - 1) / kQueryTile) * 4, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) { infini_attn_destroy(h); return INFINI_ERR_HIP; }
  *out = h;
  return INFINI_OK;
}

INFINI_EXPORT int infini_attn_destroy(infini_attn_t h) {
  if (!h) return INFINI_OK;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    if (!g_live.erase(h)) return INFINI_ERR_INVALID_ARG;
  }
  DeviceGuard dg(h->device);
  const hipError_t e = hipDeviceSynchronize();
  for (hipEvent_t ev : h->ev_pool) (void)hipEventDestroy(ev);
  (void)hipFree(h->M);   // also holds z
  (void)hipFree(h->gate);
  (void)hipFree(h->ws_base);
  if (h->layer_buf) (void)hipFree(h->layer_buf);
  if (h->dec_cache) (void)hipFree(h->dec_cache);
  if (h->dec_split) (void)hipFree(h->dec_split);
  if (h->bwd_buf) (void)hipFree(h->bwd_buf);
  if (h->mt_buf) (void)hipFree(h->mt_buf);
  if (h->zc_buf) (void)hipFree(h->zc_buf);
  if (h->split_buf) (void)hipFree(h->split_buf);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_sp) (void)hipEventDestroy(h->ev_sp);
  if (h->ev_chain) (void)hipEventDestroy(h->ev_chain);
  if (h->side) (void)hipStreamDestroy(h->side);
  delete h;
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_forward_stream(infini_attn_t h, const void* q, const void* k, const void* v,
                                             void* out, int64_t n_tokens, void* hip_stream) {
  return run_stream(h, q, k, v, out, nullptr, nullptr, n_tokens, hip_stream);
}

INFINI_EXPORT int infini_attn_forward_stream_ex(infini_attn_t h, const void* q, const void* k, const void* v,
                                                void* out, float* a_mem, float* a_dot, int64_t n_tokens,
                                                void* hip_stream) {
  return run_stream(h, q, k, v, out, a_mem, a_dot, n_tokens, hip_stream);
}

INFINI_EXPORT int infini_attn_forward_stream_local(infini_attn_t h, const void* q, const void* k,
                                                   const void* v, const void* q_local, const void* k_local,
                                                   void* out, int64_t n_tokens, void* hip_stream) {
  return run_stream(h, q, k, v, out, nullptr, nullptr, n_tokens, hip_stream, q_local, k_local);
}

INFINI_EXPORT int infini_attn_forward_stream_noalloc(infini_attn_t h, const void* q, const void* k,
                                                     const void* v, void* out, int64_t n_tokens,
                                                     void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  void* base = scratch_ptr(h->device);
  if (!base) {
    if (scratch_resolve(h->device) != hipSuccess) return INFINI_ERR_HIP;
    base = scratch_ptr(h->device);
  }
  if (n_tokens < 1) return INFINI_ERR_INVALID_ARG;
  WindowPlan plan{};
  const int rc = scratch_plan(*h, (n_tokens + h->N - 1) / h->N, base, plan);
  if (rc) return rc;
  return run_stream(h, q, k, v, out, nullptr, nullptr, n_tokens, hip_stream, nullptr, nullptr, &plan);
}

INFINI_EXPORT int infini_attn_forward_segment(infini_attn_t h, const void* q, const void* k, const void* v,
                                              void* out, int32_t n_tokens, void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (n_tokens < 1 || n_tokens > h->N) return INFINI_ERR_INVALID_ARG;
  return run_stream(h, q, k, v, out, nullptr, nullptr, n_tokens, hip_stream);
}

INFINI_EXPORT int infini_attn_reset_state(infini_attn_t h, void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  (void)hip_stream;
  h->dec_p = 0;   // an open decode segment is dropped
  // No device work: the next call that reads the state treats it as zero (the chain and
  // the state pass of its first window read 0 instead of M and z); get_state and
  // set_state write the zeros out first.
  h->state_zero = true;
  return INFINI_OK;
}

// Writes the zeros of a reset into M and z (stream-ordered), if still pending.
static hipError_t materialize_zero_state(infini_attn* h, hipStream_t st) {
  if (!h->state_zero) return hipSuccess;
  const int64_t DD = int64_t(h->D) * h->D;
  hipError_t e = zero_f32(h->M, int64_t(h->BH) * (DD + h->D), st);   // M and z
  if (e == hipSuccess && h->mt_buf) e = zero_f32(static_cast<float*>(mt_of(h, h->cur)), int64_t(h->BH) * DD / 2, st);
  if (e == hipSuccess && h->zc_buf) e = zero_f32(zc_of(h, h->cur), int64_t(h->BH) * h->D, st);
  if (e == hipSuccess) h->state_zero = false;
  return e;
}

INFINI_EXPORT int infini_attn_get_state(infini_attn_t h, float* M, float* z, void* hip_stream) {
  if (!live(h) || (!M && !z)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const size_t DD = size_t(h->D) * h->D;
  hipError_t e = join_side(h, st);
  if (e == hipSuccess) e = materialize_zero_state(h, st);
  if (e == hipSuccess && M) e = hipMemcpyAsync(M, h->M, size_t(h->BH) * DD * 4, hipMemcpyDefault, st);
  if (e == hipSuccess && z) e = hipMemcpyAsync(z, h->z, size_t(h->BH) * h->D * 4, hipMemcpyDefault, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_set_state(infini_attn_t h, const float* M, const float* z, void* hip_stream) {
  if (!live(h) || (!M && !z)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const size_t DD = size_t(h->D) * h->D;
  hipError_t e = join_side(h, st);
  if (e == hipSuccess) e = materialize_zero_state(h, st);   // a part not given keeps its (zero) value
  if (e == hipSuccess && M) e = hipMemcpyAsync(h->M, M, size_t(h->BH) * DD * 4, hipMemcpyDefault, st);
  if (e == hipSuccess && z) e = hipMemcpyAsync(h->z, z, size_t(h->BH) * h->D * 4, hipMemcpyDefault, st);
  if (e == hipSuccess && M && h->mt_buf) e = infini::launch_state_to_mt(h->M, mt_of(h, h->cur), h->BH, h->D, st);
  if (e == hipSuccess && z && h->zc_buf)
    e = hipMemcpyAsync(zc_of(h, h->cur), h->z, size_t(h->BH) * h->D * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_set_beta(infini_attn_t h, const float* beta_host) {
  if (!live(h) || !beta_host) return INFINI_ERR_INVALID_ARG;
  const int H = h->cfg.heads;
  float* gv = new (std::nothrow) float[2 * H];
  if (!gv) return INFINI_ERR_OOM;
  gate_values(beta_host, H, gv);
  DeviceGuard dg(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h->gate, gv, size_t(2) * H * 4, hipMemcpyHostToDevice);
  delete[] gv;
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int64_t infini_attn_device_bytes(infini_attn_t h) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  const int64_t DD = int64_t(h->D) * h->D;
  return int64_t(h->BH) * DD * 4 + int64_t(h->BH) * h->D * 4 + int64_t(2) * h->cfg.heads * 4 +
         static_cast<int64_t>(h->ws_bytes) + static_cast<int64_t>(h->layer_bytes) +
         (h->dec_cache ? int64_t(2) * h->BH * h->N * h->D * (h->bf16 ? 2 : 4) : 0) +
         static_cast<int64_t>(h->dec_split_bytes) +
         static_cast<int64_t>(h->bwd_bytes) + (h->mt_buf ? int64_t(2) * h->BH * DD * 2 : 0) +
         (h->zc_buf ? int64_t(2) * h->BH * h->D * 4 : 0) +
         static_cast<int64_t>(h->split_bytes);
}

INFINI_EXPORT int64_t infini_attn_window_tokens(infini_attn_t h) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  return int64_t(h->window) * h->N;
}

INFINI_EXPORT int infini_attn_profile_enable(infini_attn_t h, int enable) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  h->profiling = enable != 0;
  h->ev_used = 0;
  h->ev_marks.clear();
  return INFINI_OK;
}

INFINI_EXPORT int infini_attn_profile_read(infini_attn_t h, infini_attn_profile_t* out) {
  if (!live(h) || !out) return INFINI_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  DeviceGuard dg(h->device);
  hipError_t e = hipSuccess;
  if (h->ev_used > 0) e = hipEventSynchronize(h->ev_pool[h->ev_used - 1]);
  for (const auto& m : h->ev_marks) {
    if (e != hipSuccess) break;
    float ms = 0.f;
    e = hipEventSynchronize(h->ev_pool[m.second + 1]);   // kernels on the side stream end on their own
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, h->ev_pool[m.second], h->ev_pool[m.second + 1]);
    out->total_ms[m.first] += ms;
    out->launches[m.first] += 1;
  }
  h->ev_used = 0;
  h->ev_marks.clear();
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_project_qkv(infini_attn_t h, const void* x, const void* w_qkv, void* q, void* k,
                                          void* v, int64_t n_tokens, int32_t d_model, void* hip_stream) {
  int rc = check_layer(h, n_tokens, d_model);
  if (rc) return rc;
  if (!x || !w_qkv || !q || !k || !v) return INFINI_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_qkv, 16)) return INFINI_ERR_INVALID_ARG;
  for (const void* p : {q, k, v})
    if (!aligned(p, 8)) return INFINI_ERR_INVALID_ARG;
  const size_t x_bytes = size_t(h->cfg.batch) * size_t(n_tokens) * size_t(d_model) * 2;
  const size_t w_bytes = size_t(3) * h->cfg.heads * h->D * size_t(d_model) * 2;
  const size_t o_bytes = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * 2;
  for (const void* p : {q, k, v}) {
    if (overlaps(p, o_bytes, x, x_bytes) || overlaps(p, o_bytes, w_qkv, w_bytes)) return INFINI_ERR_INVALID_ARG;
  }
  if (overlaps(q, o_bytes, k, o_bytes) || overlaps(q, o_bytes, v, o_bytes) || overlaps(k, o_bytes, v, o_bytes))
    return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = timed(h, 4, st, [&] {
    return launch_qkv(h, x, n_tokens, 0, static_cast<int>(n_tokens), d_model, w_qkv, q, k, v, st);
  });
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_project_out(infini_attn_t h, const void* a, const void* w_o, void* out,
                                          int64_t n_tokens, int32_t d_model, void* hip_stream) {
  int rc = check_layer(h, n_tokens, d_model);
  if (rc) return rc;
  if (!a || !w_o || !out) return INFINI_ERR_INVALID_ARG;
  if (!aligned(a, 16) || !aligned(w_o, 16) || !aligned(out, 8)) return INFINI_ERR_INVALID_ARG;
  const size_t a_bytes = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * 2;
  const size_t w_bytes = size_t(d_model) * h->cfg.heads * h->D * 2;
  const size_t o_bytes = size_t(h->cfg.batch) * size_t(n_tokens) * size_t(d_model) * 2;
  if (overlaps(out, o_bytes, a, a_bytes) || overlaps(out, o_bytes, w_o, w_bytes)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = timed(h, 5, st, [&] {
    return launch_out(h, a, w_o, out, n_tokens, 0, static_cast<int>(n_tokens), d_model, st);
  });
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}

INFINI_EXPORT int infini_attn_forward_layer(infini_attn_t h, const void* x, const void* w_qkv, const void* w_o,
                                            void* out, int64_t n_tokens, int32_t d_model, void* hip_stream) {
  int rc = check_layer(h, n_tokens, d_model);
  if (rc) return rc;
  if (h->dec_p > 0) return INFINI_ERR_INVALID_ARG;
  if (!x || !w_qkv || !w_o || !out) return INFINI_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(out, 8)) return INFINI_ERR_INVALID_ARG;
  const size_t HD = size_t(h->cfg.heads) * h->D;
  const size_t x_bytes = size_t(h->cfg.batch) * size_t(n_tokens) * size_t(d_model) * 2;
  if (overlaps(out, x_bytes, x, x_bytes) || overlaps(out, x_bytes, w_qkv, 3 * HD * d_model * 2) ||
      overlaps(out, x_bytes, w_o, HD * d_model * 2))
    return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  // scratch for one window: Q, K, V, A [B, H, tc, d] bf16
  const int64_t win = int64_t(h->window) * h->N;
  const int64_t tc_max = std::min<int64_t>(win, n_tokens);
  const size_t part = size_t(h->BH) * size_t(tc_max) * size_t(h->D) * 2;
  const size_t part_al = align_up(part, 256);
  if (h->layer_bytes < 4 * part_al) {
    if (h->layer_buf) {
      if (hipStreamSynchronize(st) != hipSuccess) return INFINI_ERR_HIP;   // earlier calls may still use it
      (void)hipFree(h->layer_buf);
      h->layer_buf = nullptr;
      h->layer_bytes = 0;
    }
    if (hipMalloc(&h->layer_buf, 4 * part_al) != hipSuccess) {
      (void)hipGetLastError();
      h->layer_buf = nullptr;
      return INFINI_ERR_OOM;
    }
    h->layer_bytes = 4 * part_al;
  }
  for (int64_t t0 = 0; t0 < n_tokens; t0 += win) {
    const int tc = static_cast<int>(std::min<int64_t>(win, n_tokens - t0));
    const size_t pb = align_up(size_t(h->BH) * size_t(tc) * size_t(h->D) * 2, 256);
    char* base = static_cast<char*>(h->layer_buf);
    void *q = base, *k = base + pb, *v = base + 2 * pb, *a = base + 3 * pb;
    hipError_t e = timed(h, 4, st, [&] { return launch_qkv(h, x, n_tokens, t0, tc, d_model, w_qkv, q, k, v, st); });
    if (e != hipSuccess) return INFINI_ERR_HIP;
    rc = run_stream(h, q, k, v, a, nullptr, nullptr, tc, hip_stream);
    if (rc) return rc;
    e = timed(h, 5, st, [&] { return launch_out(h, a, w_o, out, n_tokens, t0, tc, d_model, st); });
    if (e != hipSuccess) return INFINI_ERR_HIP;
  }
  return INFINI_OK;
}

// ---- incremental decoding ------------------------------------------------------------

namespace {

// Writes the open decode segment (its n cached tokens) into M, z: the state pass and the
// chain of forward_stream over the cache as a one-segment window.
int close_decode_segment(infini_attn* h, int n, hipStream_t st) {
  const size_t es = h->bf16 ? 2 : 4;
  const char* kc = static_cast<const char*>(h->dec_cache);
  const char* vc = kc + size_t(h->BH) * h->N * h->D * es;
  infini::WindowArgs a{};
  a.q = kc;   // not read by the memory-write kernels
  a.k = kc;
  a.v = vc;
  a.q_loc = kc;
  a.k_loc = kc;
  a.B = h->cfg.batch;
  a.H = h->cfg.heads;
  a.D = h->D;
  a.T = h->N;   // the cache's row stride: N rows per (b, h)
  a.N = h->N;
  a.S = 1;
  a.n_last = n;
  a.s0 = 0;
  a.W = 1;
  a.delta = h->delta;
  a.bf16 = h->bf16;
  a.eps = h->cfg.eps;
  a.scale = h->scale;
  a.scale_log2 = static_cast<float>(double(h->scale) * 1.4426950408889634);
  a.gate_g = h->gate;
  a.gate_omg = h->gate + h->cfg.heads;
  a.M = h->M;
  a.z = h->z;
  a.ws = h->ws;
  a.zero_state = h->state_zero;
  chain_outputs(h, a);
  a.chk = chunks_for(*h, 1);
  a.ch = static_cast<int>(align_up(size_t((h->N + a.chk - 1) / a.chk), 64));
  hipError_t e = hipSuccess;
  if (h->delta) e = timed(h, 0, st, [&] { return infini::launch_key_sums(a, st); });
  if (e == hipSuccess) e = timed(h, 1, st, [&] { return infini::launch_state_pass(a, st); });
  if (e == hipSuccess) e = timed(h, 2, st, [&] { return infini::launch_chain(a, st); });
  if (e != hipSuccess) return INFINI_ERR_HIP;
  h->cur ^= 1;
  h->state_zero = false;
  return INFINI_OK;
}

}  // namespace

INFINI_EXPORT int infini_attn_decode_step(infini_attn_t h, const void* q, const void* k, const void* v, void* out,
                                          void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return INFINI_ERR_INVALID_ARG;
  for (const void* p : {q, k, v})
    if (!aligned(p, 16)) return INFINI_ERR_INVALID_ARG;
  const size_t es = h->bf16 ? 2 : 4;
  if (!aligned(out, es)) return INFINI_ERR_INVALID_ARG;
  const size_t tok_bytes = size_t(h->BH) * h->D * es;
  for (const void* p : {q, k, v})
    if (overlaps(out, tok_bytes, p, tok_bytes)) return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (join_side(h, st) != hipSuccess) return INFINI_ERR_HIP;
  if (!h->dec_cache) {
    if (hipMalloc(&h->dec_cache, 2 * size_t(h->BH) * h->N * h->D * es) != hipSuccess) {
      (void)hipGetLastError();
      h->dec_cache = nullptr;
      return INFINI_ERR_OOM;
    }
  }
  // Split keys when the (batch, head) pairs alone leave most compute units idle.
  const int nk = h->dec_p + 1;
  int nsplit = 1, chunk = 0;
  if (h->BH < kDecTargetWorkgroups && h->N > kDecChunk) {
    const int want = std::min(infini::kDecSplitMax, (kDecTargetWorkgroups + h->BH - 1) / h->BH);
    const int ns = std::min(want, (nk + kDecChunk - 1) / kDecChunk);
    if (ns > 1) {
      chunk = static_cast<int>(align_up(size_t((nk + ns - 1) / ns), kDecChunk));
      nsplit = (nk + chunk - 1) / chunk;
    }
  }
  if (nsplit > 1 && !h->dec_split) {
    const size_t part = size_t(h->BH) * infini::kDecSlots * (h->D + 2) * 4;
    const size_t bytes = part + size_t(h->BH) * 4;
    if (hipMalloc(&h->dec_split, bytes) != hipSuccess) {
      (void)hipGetLastError();
      h->dec_split = nullptr;
      return INFINI_ERR_OOM;
    }
    h->dec_split_bytes = bytes;
    // the pair counters start at zero (a fill kernel: capturable)
    if (zero_f32(h->dec_split + part / 4, h->BH, st) != hipSuccess) return INFINI_ERR_HIP;
  }
  infini::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.kc = h->dec_cache;
  a.vc = static_cast<char*>(h->dec_cache) + size_t(h->BH) * h->N * h->D * es;
  a.M = h->M;
  a.mt = mt_of(h, h->cur);
  a.z = h->z;
  a.gate_g = h->gate;
  a.gate_omg = h->gate + h->cfg.heads;
  a.B = h->cfg.batch;
  a.H = h->cfg.heads;
  a.D = h->D;
  a.N = h->N;
  a.p = h->dec_p;
  a.bf16 = h->bf16;
  a.zero_state = h->state_zero;
  a.scale_log2 = static_cast<float>(double(h->scale) * 1.4426950408889634);
  a.eps = h->cfg.eps;
  a.nsplit = nsplit;
  a.chunk = chunk;
  if (nsplit > 1) {
    a.sp_part = h->dec_split;
    a.sp_cnt = reinterpret_cast<int*>(h->dec_split + size_t(h->BH) * infini::kDecSlots * (h->D + 2));
  }
  const hipError_t e = timed(h, 6, st, [&] { return infini::launch_decode(a, st); });
  if (e != hipSuccess) return INFINI_ERR_HIP;
  if (++h->dec_p == h->N) {   // the segment is complete: write it to the memory
    h->dec_p = 0;
    return close_decode_segment(h, h->N, st);
  }
  return INFINI_OK;
}

INFINI_EXPORT int infini_attn_decode_flush(infini_attn_t h, void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (h->dec_p == 0) return INFINI_OK;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  const int n = h->dec_p;
  h->dec_p = 0;
  if (join_side(h, static_cast<hipStream_t>(hip_stream)) != hipSuccess) return INFINI_ERR_HIP;
  return close_decode_segment(h, n, static_cast<hipStream_t>(hip_stream));
}

INFINI_EXPORT int64_t infini_attn_decode_position(infini_attn_t h) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  return h->dec_p;
}

// ---- backward --------------------------------------------------------------------------

INFINI_EXPORT int infini_attn_backward(infini_attn_t h, const void* q, const void* k, const void* v,
                                       const void* d_out, const float* m0, const float* z0,
                                       const float* dm_final, const float* dz_final, float* dq, float* dk,
                                       float* dv, float* dbeta, float* dm0, float* dz0, int64_t n_tokens,
                                       void* hip_stream) {
  if (!live(h)) return INFINI_ERR_INVALID_ARG;
  if (h->dec_p > 0) return INFINI_ERR_INVALID_ARG;
  int rc = check_io(h, q, k, v, d_out, n_tokens);
  if (rc) return rc;
  if (!dq || !dk || !dv || !dbeta) return INFINI_ERR_INVALID_ARG;
  if ((m0 == nullptr) != (z0 == nullptr)) return INFINI_ERR_INVALID_ARG;
  const int64_t S64 = (n_tokens + h->N - 1) / h->N;
  if (S64 > (int64_t(1) << 30)) return INFINI_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(m0), static_cast<const void*>(z0),
                        static_cast<const void*>(dm_final), static_cast<const void*>(dz_final),
                        static_cast<const void*>(dq), static_cast<const void*>(dk), static_cast<const void*>(dv),
                        static_cast<const void*>(dbeta), static_cast<const void*>(dm0),
                        static_cast<const void*>(dz0)})
    if (!aligned(p, 4)) return INFINI_ERR_INVALID_ARG;
  const size_t es = h->bf16 ? 2 : 4;
  const size_t io_bytes = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * es;
  const size_t g_bytes = size_t(h->BH) * size_t(n_tokens) * size_t(h->D) * 4;
  for (const float* out : {dq, dk, dv})
    for (const void* in : {q, k, v, d_out})
      if (overlaps(out, g_bytes, in, io_bytes)) return INFINI_ERR_INVALID_ARG;
  if (overlaps(dq, g_bytes, dk, g_bytes) || overlaps(dq, g_bytes, dv, g_bytes) || overlaps(dk, g_bytes, dv, g_bytes))
    return INFINI_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (!dg.ok) return INFINI_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (join_side(h, st) != hipSuccess) return INFINI_ERR_HIP;   // the workspace is shared

  const int S = static_cast<int>(S64);
  // Windows of at most h->window segments: a call longer than one window first runs the
  // memory recurrence forward to record the state at every window start, then runs the
  // windows in reverse, each recomputing its forward from its recorded start state and
  // handing the gradient of that state to the window before it as its final-state
  // gradient (backpropagation through time over the whole call).
  const int Wn = static_cast<int>(std::min<int64_t>(S, h->window));
  const int nw = (S + Wn - 1) / Wn;
  const int64_t U = int64_t(Wn) * h->BH;
  const int D = h->D;
  const int pt = (h->N + 63) / 64;
  // chunks of the sigma(Q)^T dnum pass: 512-token chunks on the matrix-core path
  int rch = h->bf16 ? std::max(1, (h->N + 511) / 512)
                    : static_cast<int>(std::min<int64_t>(8, std::max<int64_t>(1, (512 + U - 1) / U)));
  const size_t rows = size_t(h->BH) * size_t(n_tokens);
  // scratch layout (256-byte aligned pieces)
  const size_t st_floats = size_t(h->BH) * (size_t(D) * D + D);   // one (M, z) state
  const size_t sz[] = {
      h->bf16 ? 256 : rows * D * es,      // 0 forward output (the bf16 recomputation writes none)
      h->bf16 ? 0 : rows * D * 4,         // 1 A_mem (the bf16 recomputation needs neither)
      h->bf16 ? 0 : rows * D * 4,         // 2 A_dot
      rows * 4, rows * 4, rows * 4, rows * 4,   // 3-6 lse, dd, den, dden
      size_t(U) * rch * D * D * 4,        // 7 rpart
      size_t(U) * rch * D * 4,            // 8 rzpart
      size_t(U) * D * D * 4,              // 9 gm
      size_t(U) * pt * D * 4,             // 10 cpart
      size_t(U) * D * 4,                  // 11 gz
      rows * 4,                           // 12 per-token gate terms
      size_t(h->BH) * D * D * 4,          // 13 state copy M
      size_t(h->BH) * D * 4,              // 14 state copy z
      h->bf16 && !h->delta ? size_t(U) * D * D * 4 : 0,   // 15 G_s packed in bf16, two orientations
      nw > 1 ? size_t(nw) * st_floats * 4 : 0,             // 16 the state at every window start
      nw > 1 ? 2 * st_floats * 4 : 0,                      // 17 state gradients between windows
  };
  constexpr int NP = sizeof(sz) / sizeof(sz[0]);
  size_t total = 0;
  for (size_t x : sz) total += align_up(x, 256);
  if (h->bwd_bytes < total) {
    if (h->bwd_buf) {
      if (hipStreamSynchronize(st) != hipSuccess) return INFINI_ERR_HIP;
      (void)hipFree(h->bwd_buf);
      h->bwd_buf = nullptr;
      h->bwd_bytes = 0;
    }
    if (hipMalloc(&h->bwd_buf, total) != hipSuccess) {
      (void)hipGetLastError();
      h->bwd_buf = nullptr;
      return INFINI_ERR_OOM;
    }
    h->bwd_bytes = total;
  }
  void* part[NP];
  {
    char* p = static_cast<char*>(h->bwd_buf);
    for (int i = 0; i < NP; ++i) {
      part[i] = p;
      p += align_up(sz[i], 256);
    }
  }
  float* Ms = static_cast<float*>(part[13]);   // M then z: one (M, z) state
  float* zs = static_cast<float*>(part[14]);
  const int64_t DDl = int64_t(D) * D;
  hipError_t e = hipSuccess;
  if (m0) {
    e = hipMemcpyAsync(Ms, m0, sz[13], hipMemcpyDefault, st);
    if (e == hipSuccess) e = hipMemcpyAsync(zs, z0, sz[14], hipMemcpyDefault, st);
    if (e != hipSuccess) return INFINI_ERR_HIP;
  }

  // the forward of a window, keeping the backward's per-token terms (or A_mem, A_dot) and
  // the per-segment states in the workspace; the handle's own state is not touched
  infini::WindowArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_loc = q;
  a.k_loc = k;
  a.out = part[0];
  a.lse = static_cast<float*>(part[3]);
  if (h->bf16) {   // the attention writes the backward's per-token terms directly
    a.bwd_dout = d_out;
    a.bwd_dd = static_cast<float*>(part[4]);
    a.bwd_den = static_cast<float*>(part[5]);
    a.bwd_dden = static_cast<float*>(part[6]);
    a.bwd_bq = static_cast<float*>(part[12]);
  } else {
    a.a_mem = static_cast<float*>(part[1]);
    a.a_dot = static_cast<float*>(part[2]);
  }
  a.B = h->cfg.batch;
  a.H = h->cfg.heads;
  a.D = D;
  a.T = n_tokens;
  a.N = h->N;
  a.S = S;
  a.n_last = static_cast<int>(n_tokens - int64_t(S - 1) * h->N);
  a.delta = h->delta;
  a.bf16 = h->bf16;
  a.eps = h->cfg.eps;
  a.scale = h->scale;
  a.scale_log2 = static_cast<float>(double(h->scale) * 1.4426950408889634);
  a.gate_g = h->gate;
  a.gate_omg = h->gate + h->cfg.heads;
  a.M = Ms;
  a.z = zs;
  a.ws = h->ws;
  auto set_window = [&](int w) {
    a.s0 = w * Wn;
    a.W = std::min(Wn, S - a.s0);
    a.chk = chunks_for(*h, a.W);
    a.ch = static_cast<int>(align_up(size_t((h->N + a.chk - 1) / a.chk), 64));
  };
  // state pass and chain of the window set in a: the chain leaves the window's final state
  // in (Ms, zs) and records every segment's M^T_{s-1}, z_{s-1}
  auto recurrence = [&](bool zero) -> hipError_t {
    a.zero_state = zero;
    hipError_t er = hipSuccess;
    if (h->delta) er = timed(h, 0, st, [&] { return infini::launch_key_sums(a, st); });
    if (er == hipSuccess) er = timed(h, 1, st, [&] { return infini::launch_state_pass(a, st); });
    if (er == hipSuccess) er = timed(h, 2, st, [&] { return infini::launch_chain(a, st); });
    a.zero_state = false;
    return er;
  };
  float* ckpt = nw > 1 ? static_cast<float*>(part[16]) : nullptr;
  float* gbuf = nw > 1 ? static_cast<float*>(part[17]) : nullptr;
  // Ms holds M and zs holds z; a recorded state is M then z, st_floats in all
  auto save_state = [&](float* dst) -> hipError_t {
    hipError_t er = hipMemcpyAsync(dst, Ms, sz[13], hipMemcpyDeviceToDevice, st);
    if (er == hipSuccess) er = hipMemcpyAsync(dst + h->BH * DDl, zs, sz[14], hipMemcpyDeviceToDevice, st);
    return er;
  };
  auto load_state = [&](const float* src) -> hipError_t {
    hipError_t er = hipMemcpyAsync(Ms, src, sz[13], hipMemcpyDeviceToDevice, st);
    if (er == hipSuccess) er = hipMemcpyAsync(zs, src + h->BH * DDl, sz[14], hipMemcpyDeviceToDevice, st);
    return er;
  };
  if (nw > 1) {   // the state at every window start
    if (!m0) e = zero_f32(Ms, int64_t(h->BH) * DDl, st);
    if (!m0 && e == hipSuccess) e = zero_f32(zs, int64_t(h->BH) * D, st);
    for (int w = 0; w < nw && e == hipSuccess; ++w) {
      e = save_state(ckpt + size_t(w) * st_floats);
      if (e == hipSuccess && w + 1 < nw) {
        set_window(w);
        e = recurrence(false);
      }
    }
    if (e != hipSuccess) return INFINI_ERR_HIP;
  }

  infini::BackwardArgs bw{};
  bw.dout = d_out;
  bw.dd = static_cast<float*>(part[4]);
  bw.den = static_cast<float*>(part[5]);
  bw.dden = static_cast<float*>(part[6]);
  bw.dq = dq;
  bw.dk = dk;
  bw.dv = dv;
  bw.rpart = static_cast<float*>(part[7]);
  bw.rzpart = static_cast<float*>(part[8]);
  bw.gm = static_cast<float*>(part[9]);
  bw.cpart = static_cast<float*>(part[10]);
  bw.gz = static_cast<float*>(part[11]);
  bw.gpk = sz[15] ? static_cast<uint16_t*>(part[15]) : nullptr;
  bw.bq = static_cast<float*>(part[12]);
  bw.dbeta = dbeta;
  bw.rch = rch;
  bw.pt = pt;
  bw.ct = h->bf16 ? (h->N + 127) / 128 : pt;   // the bf16 update kernel works on 128-token tiles
  bw.skip_dbeta = nw > 1;
  for (int w = nw - 1; w >= 0 && e == hipSuccess; --w) {
    set_window(w);
    if (nw > 1) e = load_state(ckpt + size_t(w) * st_floats);
    if (e == hipSuccess) e = recurrence(nw == 1 && m0 == nullptr);
    if (e == hipSuccess) e = timed(h, 3, st, [&] { return infini::launch_attention(a, st); });
    if (e != hipSuccess) break;
    bw.w = a;
    bw.w.zero_state = false;
    // gradient of this window's final state: the caller's for the last window, else what
    // the next window handed back; the gradient of its start state goes to the window
    // before it (or to the caller's dm0, dz0)
    float* gnext = gbuf ? gbuf + size_t((w + 1) & 1) * st_floats : nullptr;
    float* gmine = gbuf ? gbuf + size_t(w & 1) * st_floats : nullptr;
    bw.dm_final = w == nw - 1 ? dm_final : gnext;
    bw.dz_final = w == nw - 1 ? dz_final : gnext + h->BH * DDl;
    bw.dm0 = w == 0 ? dm0 : gmine;
    bw.dz0 = w == 0 ? dz0 : gmine + h->BH * DDl;
    e = timed(h, 7, st, [&] { return infini::launch_backward(bw, st); });
  }
  if (e == hipSuccess && nw > 1) {
    bw.w.s0 = 0;
    bw.w.W = S;
    e = timed(h, 7, st, [&] { return infini::launch_bwd_dbeta(bw, st); });
  }
  return e == hipSuccess ? INFINI_OK : INFINI_ERR_HIP;
}
