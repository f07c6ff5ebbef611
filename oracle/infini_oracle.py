"""Infini-attention layer forward: the CPU oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it.

What it is: the plain definition of one Infini-attention layer's forward pass, in
numpy float64, one (batch, head) pair at a time, one segment after the other.  No
blocking, fusion or reordering beyond what the equations state.

Source of every formula: the architecture summary of "Leave No Context Behind:
Efficient Infinite Context Transformers with Infini-attention" (arXiv 2404.07143) on
paper-graph-ui.vercel.app, section 3.4 "Detailed, Sentence-Based Technical
Breakdown".  Equation numbers are the ones that page uses in its prose:

* Eq. 4  -- the recurrent layer contract  O_s, M_s = infini-attention(X_s, M_{s-1})
* Eq. 6  -- local causal dot-product attention inside the segment
* Eq. 7  -- memory retrieval  A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1})
* Eq. 8  -- linear memory update  M_s = M_{s-1} + sigma(K)^T V,  z_s = z_{s-1} + sum_t sigma(K_t)
* Eq. 9  -- delta-rule update  M_s = M_{s-1} + sigma(K)^T (V - sigma(K)M_{s-1}/(sigma(K)z_{s-1}))
* Eq. 10 -- per-head gate  A = sigmoid(beta) A_mem + (1 - sigmoid(beta)) A_dot

Readings taken where the page is silent or loose:

1. Softmax scale: the page prints 1/sqrt(d_model) but also says the local attention is
   vanilla per-head attention.  The scale is an explicit argument; ``None`` means
   1/sqrt(d) with d the per-head dimension.
2. eps: the page's retrieval has no epsilon, so segment 0 would be 0/0.  Here the
   denominator is sigma(.) z + eps, in Eq. 7 and in Eq. 9's retrieved value alike.
   Segment 0 therefore retrieves exactly 0 from the zero memory.
3. ELU alpha = 1 (the default of the cited ELU paper): sigma(x) = x + 1 for x > 0 and
   exp(x) for x <= 0.
4. The same (position-embedding free) Q and K feed both the local and the memory path.
5. Eq. 9 is applied per segment: the retrieved value for every token of segment s uses
   M_{s-1} and z_{s-1}; z is updated as in Eq. 8.
6. beta is a logit, one per head, shared by the batch and all tokens.
7. Every batch element carries its own M and z.
8. The final segment of a stream may be shorter than N (the summary's BookSum
   discussion of 500K tokens in 2048-token segments); it is processed with its own length.
9. The projections around the heads (section "Standard Dot-Product Attention", Query,
   Key, Value projections, Eq. 5; section "Multi-Head Infini-Attention", Eq. 11) take
   the weights in the "out x in" layout: W_qkv [3 H d, d_model] holds, in its rows
   h*d + j, H*d + h*d + j and 2*H*d + h*d + j, column j of head h's W_Q, W_K and W_V;
   W_o [d_model, H d] is the transpose of the page's W_O, so column h*d + j multiplies
   feature j of head h, heads concatenated in order.  ``layer_forward`` can round Q, K,
   V and the head outputs to bfloat16 between the steps (``bf16_between``), the storage
   precision of a bf16 layer; everything else stays float64.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "elu_plus_one",
    "sigmoid",
    "local_causal_attention",
    "memory_retrieval",
    "memory_update_linear",
    "memory_update_delta",
    "gate",
    "segment_forward",
    "forward",
    "segment_bounds",
    "state_numbers_per_layer",
    "advance",
    "round_to_bf16",
    "project_qkv",
    "project_out",
    "layer_forward",
    "decode_token",
    "decode_stream",
]

LINEAR = "linear"
DELTA = "delta"


def elu_plus_one(x):
    """sigma = ELU + 1, element-wise (section "Compressive Memory", text under Eq. 7).

    ELU with alpha = 1: x for x > 0, exp(x) - 1 otherwise; adding one gives x + 1 and
    exp(x).  The feature map is strictly positive.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def sigmoid(beta):
    """The logistic function of the gate logit (section "The Gating Mechanism", Eq. 10).

    Written in the two-branch form so that sigmoid(-inf) = 0 and sigmoid(+inf) = 1 exactly.
    """
    b = np.asarray(beta, dtype=np.float64)
    out = np.empty_like(b)
    pos = b >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-b[pos]))
    e = np.exp(b[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def local_causal_attention(q, k, v, scale):
    """Eq. 6: A_dot = softmax(scale * Q K^T, causal) V inside one segment.

    q, k: [n, d_key]; v: [n, d_value].  Row i attends to positions j <= i of the same
    segment only (section "Standard Dot-Product Attention").  Row-wise softmax with
    the row maximum subtracted first.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    scores = scale * (q @ k.T)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    scores = scores - scores.max(axis=1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def memory_retrieval(q, M, z, eps):
    """Eq. 7: A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps).

    q: [n, d_key]; M: [d_key, d_value]; z: [d_key].  The denominator is one scalar per
    query row.  eps is reading 2 of the module docstring.
    """
    sq = elu_plus_one(q)
    num = sq @ np.asarray(M, dtype=np.float64)
    den = sq @ np.asarray(z, dtype=np.float64) + eps
    return num / den[:, None]


def memory_update_linear(k, v, M, z):
    """Eq. 8: M_s = M_{s-1} + sigma(K)^T V;  z_s = z_{s-1} + sum_t sigma(K_t)."""
    sk = elu_plus_one(k)
    v = np.asarray(v, dtype=np.float64)
    return (np.asarray(M, dtype=np.float64) + sk.T @ v,
            np.asarray(z, dtype=np.float64) + sk.sum(axis=0))


def memory_update_delta(k, v, M, z, eps):
    """Eq. 9: subtract what the memory already returns for sigma(K), then bind.

    The retrieved value uses the state from before the segment (M_{s-1}, z_{s-1}) for
    every token; z follows Eq. 8 (the page: the delta rule keeps "the same
    normalization term" as the linear one).
    """
    sk = elu_plus_one(k)
    v = np.asarray(v, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    retrieved = (sk @ M) / (sk @ z + eps)[:, None]
    return M + sk.T @ (v - retrieved), z + sk.sum(axis=0)


def gate(a_mem, a_dot, beta):
    """Eq. 10: A = sigmoid(beta) A_mem + (1 - sigmoid(beta)) A_dot, beta a scalar."""
    g = float(sigmoid(np.array([beta]))[0])
    return g * np.asarray(a_mem, dtype=np.float64) + (1.0 - g) * np.asarray(a_dot, dtype=np.float64)


def segment_forward(q, k, v, M, z, beta, update, eps, scale, q_local=None, k_local=None):
    """Eq. 4 for one head and one segment: returns (A, M_s, z_s, A_mem, A_dot).

    Order as the page states it: read the memory with the previous state, compute the
    local attention, gate the two, then write the memory.  ``q_local`` / ``k_local``
    (default: q / k) are the query and key of the local attention only, e.g. with
    position embeddings, which the page's training notes apply to the local arm after
    the memory read and update; the memory always uses the PE-free q / k.
    """
    a_mem = memory_retrieval(q, M, z, eps)
    a_dot = local_causal_attention(q if q_local is None else q_local,
                                   k if k_local is None else k_local, v, scale)
    a = gate(a_mem, a_dot, beta)
    if update == LINEAR:
        M_new, z_new = memory_update_linear(k, v, M, z)
    elif update == DELTA:
        M_new, z_new = memory_update_delta(k, v, M, z, eps)
    else:
        raise ValueError(f"unknown update rule {update!r}")
    return a, M_new, z_new, a_mem, a_dot


def segment_bounds(n_tokens, segment_len):
    """Segment chunking (section "Training Infrastructure"): [start, stop) per segment.

    ceil(n_tokens / N) segments; all have N tokens except possibly the last.
    """
    if segment_len < 1:
        raise ValueError("segment_len must be >= 1")
    return [(s, min(s + segment_len, n_tokens)) for s in range(0, n_tokens, segment_len)]


def state_numbers_per_layer(heads, d_key, d_value):
    """Numbers held by one layer's compressive memory (section "Multi-Head Infini-Attention",
    memory footprint): H * d_key * d_value for M plus H * d_key for z."""
    return heads * d_key * d_value, heads * d_key


def forward(Q, K, V, beta, segment_len, update=LINEAR, eps=1e-6, scale=None,
            M0=None, z0=None, return_parts=False, Q_local=None, K_local=None):
    """The layer over a whole stream.

    Q, K, V: [B, H, L, d] (any real dtype; upcast to float64).  beta: [H].
    Q_local, K_local: optional [B, H, L, d] query / key of the local attention (see
    ``segment_forward``); the memory path uses Q and K.
    M0: [B, H, d, d] and z0: [B, H, d] initial state (zeros when None).
    Returns (O [B,H,L,d], M [B,H,d,d], z [B,H,d]) and, with ``return_parts``, also
    A_mem and A_dot [B,H,L,d].  Each (b, h) is an independent chain (section
    "Multi-Head Infini-Attention": heads run in parallel with no communication).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Ql = None if Q_local is None else np.asarray(Q_local, dtype=np.float64)
    Kl = None if K_local is None else np.asarray(K_local, dtype=np.float64)
    B, H, L, d = Q.shape
    dv = V.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    beta = np.asarray(beta, dtype=np.float64).reshape(H)
    M = np.zeros((B, H, d, dv)) if M0 is None else np.array(M0, dtype=np.float64)
    z = np.zeros((B, H, d)) if z0 is None else np.array(z0, dtype=np.float64)
    O = np.empty((B, H, L, dv))
    A_mem = np.empty((B, H, L, dv)) if return_parts else None
    A_dot = np.empty((B, H, L, dv)) if return_parts else None
    bounds = segment_bounds(L, segment_len)
    for b in range(B):
        for h in range(H):
            Mbh, zbh = M[b, h], z[b, h]
            for lo, hi in bounds:
                a, Mbh, zbh, am, ad = segment_forward(
                    Q[b, h, lo:hi], K[b, h, lo:hi], V[b, h, lo:hi], Mbh, zbh,
                    beta[h], update, eps, scale,
                    None if Ql is None else Ql[b, h, lo:hi], None if Kl is None else Kl[b, h, lo:hi])
                O[b, h, lo:hi] = a
                if return_parts:
                    A_mem[b, h, lo:hi] = am
                    A_dot[b, h, lo:hi] = ad
            M[b, h], z[b, h] = Mbh, zbh
    if return_parts:
        return O, M, z, A_mem, A_dot
    return O, M, z


def advance(k, v, M, z, update, eps):
    """One step of the memory recurrence alone (Eq. 8 or Eq. 9) for one segment.

    A segment's output depends only on its own Q/K/V and the state before it, so a
    long stream can be checked on a sample of segments by advancing the state with
    this and calling ``segment_forward`` only where outputs are wanted.
    """
    if update == LINEAR:
        return memory_update_linear(k, v, M, z)
    if update == DELTA:
        return memory_update_delta(k, v, M, z, eps)
    raise ValueError(f"unknown update rule {update!r}")


def round_to_bf16(x):
    """Round to the nearest bfloat16 value (ties to even), kept as float64.

    bfloat16 has 8 significant bits: with x = m 2^e, 1/2 <= |m| < 1, the result is
    round(256 m) 2^(e - 8) (both scalings by powers of two are exact).  Infinities and
    NaN pass through; bfloat16 overflow and subnormals are not modelled.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.round(m * 256.0), e - 8)   # np.round: ties to even
    return np.where(np.isfinite(x), r, x)


def project_qkv(X, W_qkv, heads, head_dim):
    """Eq. 5 for every head: Q_h = X W_Q^(h), K_h = X W_K^(h), V_h = X W_V^(h).

    X: [B, L, d_model]; W_qkv: [3 H d, d_model] ("out x in", reading 9).
    Returns Q, K, V as [B, H, L, d] float64.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W_qkv, dtype=np.float64)
    B, L, _ = X.shape
    H, d = heads, head_dim
    Y = X @ W.T   # [B, L, 3 H d]: feature p*H*d + h*d + j
    parts = []
    for p in range(3):
        blk = Y[:, :, p * H * d:(p + 1) * H * d].reshape(B, L, H, d)
        parts.append(blk.transpose(0, 2, 1, 3))
    return tuple(parts)


def project_out(A, W_o):
    """Eq. 11: O = [A_1; ...; A_H] W_O, the head outputs concatenated along features.

    A: [B, H, L, d]; W_o: [d_model, H d] (the page's W_O transposed, reading 9).
    Returns O as [B, L, d_model] float64.
    """
    A = np.asarray(A, dtype=np.float64)
    W = np.asarray(W_o, dtype=np.float64)
    B, H, L, d = A.shape
    cat = A.transpose(0, 2, 1, 3).reshape(B, L, H * d)   # [A_1; ...; A_H] per token
    return cat @ W.T


def layer_forward(X, W_qkv, W_o, beta, segment_len, heads, head_dim, update=LINEAR, eps=1e-6,
                  scale=None, M0=None, z0=None, bf16_between=False):
    """The whole layer on a stream X [B, L, d_model]: Eq. 5, the per-head recurrence
    (Eq. 4, 6-10, ``forward``), Eq. 11.  Returns (O [B, L, d_model], M, z)."""
    Q, K, V = project_qkv(X, W_qkv, heads, head_dim)
    if bf16_between:
        Q, K, V = round_to_bf16(Q), round_to_bf16(K), round_to_bf16(V)
    A, M, z = forward(Q, K, V, beta, segment_len, update, eps, scale, M0, z0)
    if bf16_between:
        A = round_to_bf16(A)
    return project_out(A, W_o), M, z


def decode_token(q, k, v, cache_k, cache_v, M, z, beta, eps, scale):
    """One token of incremental decoding for one head (the summary's "fast streaming
    inference": tokens arrive one at a time inside a segment).

    The token's key and value join the segment's cache; the local attention (Eq. 6) is a
    softmax over every cached token, all of which precede or are the current one; the
    memory read (Eq. 7) uses the state from before the segment; Eq. 10 gates the two.
    q, k, v: [d]; cache_k, cache_v: [n, d], the segment's earlier tokens.
    Returns (a [d], cache_k', cache_v').
    """
    q = np.asarray(q, dtype=np.float64)
    ck = np.vstack([np.asarray(cache_k, dtype=np.float64).reshape(-1, q.shape[0]),
                    np.asarray(k, dtype=np.float64)[None]])
    cv = np.vstack([np.asarray(cache_v, dtype=np.float64).reshape(-1, np.asarray(v).shape[0]),
                    np.asarray(v, dtype=np.float64)[None]])
    s = scale * (ck @ q)
    w = np.exp(s - s.max())
    a_dot = (w @ cv) / w.sum()
    a_mem = memory_retrieval(q[None], M, z, eps)[0]
    return gate(a_mem, a_dot, beta), ck, cv


def decode_stream(Q, K, V, beta, segment_len, update=LINEAR, eps=1e-6, scale=None, M0=None, z0=None,
                  flush=True):
    """A stream fed one token at a time through ``decode_token``.

    The memory is written (Eq. 8 / Eq. 9 over the cached segment, ``advance``) when the
    cache holds segment_len tokens, and, with ``flush``, once more for a partial last
    segment.  Q, K, V: [B, H, L, d].  Returns (O [B, H, L, d], M, z, open_tokens), where
    open_tokens is the number of cached tokens not yet written to the memory.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, L, d = Q.shape
    dv = V.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    beta = np.asarray(beta, dtype=np.float64).reshape(H)
    M = np.zeros((B, H, d, dv)) if M0 is None else np.array(M0, dtype=np.float64)
    z = np.zeros((B, H, d)) if z0 is None else np.array(z0, dtype=np.float64)
    O = np.empty((B, H, L, dv))
    open_tokens = 0
    for b in range(B):
        for h in range(H):
            ck, cv = np.zeros((0, d)), np.zeros((0, dv))
            for t in range(L):
                O[b, h, t], ck, cv = decode_token(Q[b, h, t], K[b, h, t], V[b, h, t], ck, cv, M[b, h], z[b, h],
                                                  beta[h], eps, scale)
                if ck.shape[0] == segment_len:
                    M[b, h], z[b, h] = advance(ck, cv, M[b, h], z[b, h], update, eps)
                    ck, cv = np.zeros((0, d)), np.zeros((0, dv))
            if flush and ck.shape[0] > 0:
                M[b, h], z[b, h] = advance(ck, cv, M[b, h], z[b, h], update, eps)
                ck = np.zeros((0, d))
            open_tokens = ck.shape[0]
    return O, M, z, open_tokens
