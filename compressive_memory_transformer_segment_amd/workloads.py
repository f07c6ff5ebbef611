"""Seeded synthetic inputs shaped like the Infini-attention workloads.

This module holds input generation only: random draws, the bf16 rounding of inputs,
the per-token scale and the planted key/value pair.  None of the layer's arithmetic
lives here.  It is the one module that both the GPU tests/bench and the CPU oracle
side use, so both see bit-identical inputs.

The shapes follow the architecture summary of "Leave No Context Behind" (arXiv
2404.07143): per-head dimension 128 and 2048-token segments (section 3.4, "Standard
Dot-Product Attention" and "Training Infrastructure"), 8 heads per layer, streams of
32K tokens (16 segments) and of 500K-1M tokens (the passkey and book-summary
experiments).  The pages' data sets (PG19, passkey text, BookSum) and trained weights
are not available; these draws stand in for them.

Recipe (fixed, so any segment of any stream can be regenerated on its own):
* every (seed, batch index, segment index, tensor id, head) gets its own
  ``numpy.random.SeedSequence``; tensor ids: 0 = Q, 1 = K, 2 = V, 3 = per-token scale
  (drawn once per (seed, batch, segment), head slot 0);
* Q, K, V entries are N(0, 1) / sqrt(d), drawn as float32, [n, d] per head;
* a per-token scale exp(U(ln 0.5, ln 2)), one per (batch, token), multiplies Q, K and V
  of every head before rounding (the 32-head, 512K-token workload);
* bf16 workloads round the float32 draws to bf16 with round-to-nearest-even;
* beta ~ N(0, 1) per head from SeedSequence([seed, BETA_TAG]), or 0;
* the planted pair (1M-token workload): k* = g / ||g|| with g ~ N(0, I_d), normalised
  in float64 and then rounded; v* ~ N(0, 1) / sqrt(d).  It replaces K and V at token 0
  of segment 0 in every head, and Q at the stream's final token is k*;
* the whole layer (input X and the projection weights, section "Standard Dot-Product
  Attention" and "Multi-Head Infini-Attention"): X [B, L, d_model] ~ N(0, 1) per entry,
  W_qkv [3 H d, d_model] ~ N(0, 1 / (d_model d)) so that the projected Q, K, V have the
  N(0, 1) / sqrt(d) entries of the per-head workloads, W_o [d_model, H d] ~ N(0, 1 / (H d));
  drawn as float32 from SeedSequence([seed, LAYER_TAG, tensor id]) (X per batch element:
  [seed, LAYER_TAG, 0, b]) and rounded to bf16.  d_model = H d unless stated (the pages'
  small models: 8 heads of 128 in d_model = 1024).
"""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

BETA_TAG = 0xBE7A
PLANT_TAG = 0x9A55
LAYER_TAG = 0x1A7E

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_SCALE = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    segment_len: int
    n_tokens: int
    io_dtype: str          # "bf16" or "f32"
    update: str            # "linear" or "delta"
    seed: int
    beta: str = "normal"   # "normal" (N(0,1) per head) or "zero"
    token_scale: bool = False
    plant: bool = False
    eps: float = 1e-6

    @property
    def n_segments(self) -> int:
        return -(-self.n_tokens // self.segment_len)

    def segment_len_of(self, s: int) -> int:
        return min(self.segment_len, self.n_tokens - s * self.segment_len)

    def with_tokens(self, n_tokens: int, name: str | None = None) -> "Workload":
        return dataclasses.replace(self, n_tokens=n_tokens, name=name or f"{self.name}@{n_tokens}")

    def with_batch(self, batch: int) -> "Workload":
        return dataclasses.replace(self, batch=batch, name=f"{self.name}-b{batch}")


# The five workloads, named by what they are.
WORKLOADS = {
    w.name: w
    for w in [
        # one head, d=64, 64-token segments, 4 segments, fp32 I/O, beta = 0
        Workload("tiny-f32-h1-d64-n64-l256-linear", 1, 1, 64, 64, 256, "f32", "linear", 0,
                 beta="zero"),
        # 8 heads, d=128, 2048-token segments, 32K tokens: the throughput workload
        Workload("h8-d128-n2048-l32k-linear", 1, 8, 128, 2048, 32768, "bf16", "linear", 1),
        Workload("h8-d128-n2048-l32k-delta", 1, 8, 128, 2048, 32768, "bf16", "delta", 2),
        Workload("b4-h8-d128-n2048-l32k-delta", 4, 8, 128, 2048, 32768, "bf16", "delta", 2),
        # 8B-like layer: 32 heads, 256 segments, per-token scale, delta rule
        Workload("h32-d128-n2048-l512k-delta-scaled", 1, 32, 128, 2048, 524288, "bf16", "delta", 3,
                 token_scale=True),
        # 1M-token stream with a planted key/value pair
        Workload("h8-d128-n2048-l1m-linear-planted", 1, 8, 128, 2048, 1048576, "bf16", "linear", 4,
                 plant=True),
    ]
}

THROUGHPUT_WORKLOAD = "h8-d128-n2048-l32k-linear"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def beta_for(w: Workload) -> np.ndarray:
    if w.beta == "zero":
        return np.zeros(w.heads, dtype=np.float32)
    return _rng(w.seed, BETA_TAG).standard_normal(w.heads).astype(np.float32)


def planted_pair(w: Workload):
    """(k*, v*) as float32 rows of length d (bf16-representable for bf16 workloads)."""
    g = _rng(w.seed, PLANT_TAG, 0).standard_normal(w.head_dim)
    k_star = (g / np.linalg.norm(g)).astype(np.float32)
    v_star = (_rng(w.seed, PLANT_TAG, 1).standard_normal(w.head_dim) / math.sqrt(w.head_dim)).astype(np.float32)
    if w.io_dtype == "bf16":
        k_star, v_star = round_to_bf16(k_star), round_to_bf16(v_star)
    return k_star, v_star


def layer_inputs(w: Workload, d_model: int | None = None):
    """(X [B, L, d_model], W_qkv [3 H d, d_model], W_o [d_model, H d]) as float32 arrays
    holding bf16 values (the recipe above)."""
    H, d = w.heads, w.head_dim
    dm = H * d if d_model is None else d_model
    X = np.empty((w.batch, w.n_tokens, dm), dtype=np.float32)
    for b in range(w.batch):
        X[b] = _rng(w.seed, LAYER_TAG, 0, b).standard_normal((w.n_tokens, dm), dtype=np.float32)
    w_qkv = _rng(w.seed, LAYER_TAG, 1).standard_normal((3 * H * d, dm), dtype=np.float32) / np.float32(
        math.sqrt(dm * d))
    w_o = _rng(w.seed, LAYER_TAG, 2).standard_normal((dm, H * d), dtype=np.float32) / np.float32(math.sqrt(H * d))
    return round_to_bf16(X), round_to_bf16(w_qkv), round_to_bf16(w_o)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        _POOL = concurrent.futures.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def segment_inputs(w: Workload, b: int, s: int, plant: bool | None = None, heads=None):
    """Q, K, V of batch element b, segment s: three float32 arrays [len(heads), n, d].

    ``heads`` selects a subset of heads (default: all); each head's draws depend only on
    (seed, b, s, tensor, head), so a subset equals the same rows of the full draw.
    """
    n = w.segment_len_of(s)
    if n <= 0:
        raise ValueError(f"segment {s} is past the end of a {w.n_tokens}-token stream")
    heads = list(range(w.heads)) if heads is None else list(heads)
    inv = np.float32(1.0 / math.sqrt(w.head_dim))
    scale = None
    if w.token_scale:
        lo, hi = math.log(0.5), math.log(2.0)
        scale = np.exp(_rng(w.seed, b, s, TENSOR_SCALE, 0).uniform(lo, hi, size=n)).astype(np.float32)
    qkv = [np.empty((len(heads), n, w.head_dim), dtype=np.float32) for _ in range(3)]

    def draw(job):
        t, i = job
        x = _rng(w.seed, b, s, t, heads[i]).standard_normal((n, w.head_dim), dtype=np.float32) * inv
        if scale is not None:
            x = x * scale[:, None]
        if w.io_dtype == "bf16":
            x = round_to_bf16(x)
        qkv[t][i] = x

    jobs = [(t, i) for t in (TENSOR_Q, TENSOR_K, TENSOR_V) for i in range(len(heads))]
    if len(heads) * n * w.head_dim >= (1 << 18):
        list(_pool().map(draw, jobs))
    else:
        for job in jobs:
            draw(job)
    if (w.plant if plant is None else plant):
        k_star, v_star = planted_pair(w)
        q, k, v = qkv
        if s == 0:
            k[:, 0, :] = k_star
            v[:, 0, :] = v_star
        if s == w.n_segments - 1:
            q[:, n - 1, :] = k_star
    return tuple(qkv)


def stream_inputs(w: Workload, plant: bool | None = None):
    """Whole-stream Q, K, V as float32 [B, H, L, d] (keep to small workloads)."""
    shape = (w.batch, w.heads, w.n_tokens, w.head_dim)
    Q, K, V = (np.empty(shape, dtype=np.float32) for _ in range(3))
    for b in range(w.batch):
        for s in range(w.n_segments):
            lo = s * w.segment_len
            q, k, v = segment_inputs(w, b, s, plant=plant)
            n = q.shape[1]
            Q[b, :, lo:lo + n], K[b, :, lo:lo + n], V[b, :, lo:lo + n] = q, k, v
    return Q, K, V
