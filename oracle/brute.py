"""Pure-Python scalar-loop versions of the Infini-attention quantities (tiny inputs).

TEST INFRASTRUCTURE.  Used only by ``tests/`` to pin ``oracle.infini_oracle`` against a
second writing that shares none of its code: lists and ``math`` only, no numpy, one
multiply-add at a time.  Source of the formulas: the architecture summary of "Leave No
Context Behind" (arXiv 2404.07143, paper-graph-ui.vercel.app), section 3.4.

Where a quantity has a closed form that differs from the recurrence (the retrieval of
the linear rule is linearised attention over the whole history, section "Compressive
Memory", the expansion of M_{s-1} as a sum of outer products), the closed form is what
is written here, so the two sides compute it by different routes.
"""

import math


def sigma(x):
    """ELU(x) + 1 with alpha = 1."""
    return x + 1.0 if x > 0.0 else math.exp(x)


def dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def causal_softmax_row(q_row, keys, values, scale):
    """One output row of Eq. 6: weights over keys[0..i] (the caller passes the prefix)."""
    scores = [scale * dot(q_row, k) for k in keys]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    dv = len(values[0])
    out = [0.0] * dv
    for wj, vj in zip(w, values):
        for c in range(dv):
            out[c] += wj * vj[c]
    return [o / tot for o in out]


def local_attention(q, k, v, scale):
    """Eq. 6 for one segment, row by row."""
    return [causal_softmax_row(q[i], k[: i + 1], v[: i + 1], scale) for i in range(len(q))]


def retrieval_from_history(q_row, hist_k, hist_v, eps):
    """Linear rule only: A_mem for one query as linearised attention over every earlier
    token, sum_t (sigma(q).sigma(k_t)) v_t / (sum_t sigma(q).sigma(k_t) + eps).
    With no history the numerator is an empty sum, so the result is 0."""
    sq = [sigma(x) for x in q_row]
    dv = len(hist_v[0]) if hist_v else len(q_row)
    num = [0.0] * dv
    den = 0.0
    for k_t, v_t in zip(hist_k, hist_v):
        w = dot(sq, [sigma(x) for x in k_t])
        den += w
        for c in range(dv):
            num[c] += w * v_t[c]
    return [x / (den + eps) for x in num]


def state_from_history(hist_k, hist_v, d, dv):
    """Linear rule only: M = sum_t sigma(k_t)^T v_t and z = sum_t sigma(k_t), entry by entry."""
    M = [[0.0] * dv for _ in range(d)]
    z = [0.0] * d
    for k_t, v_t in zip(hist_k, hist_v):
        sk = [sigma(x) for x in k_t]
        for i in range(d):
            z[i] += sk[i]
            for j in range(dv):
                M[i][j] += sk[i] * v_t[j]
    return M, z


def delta_step(k, v, M, z, eps):
    """Eq. 9 for one segment with explicit loops, from the pre-segment state."""
    d = len(M)
    dv = len(M[0])
    sks = [[sigma(x) for x in row] for row in k]
    new_M = [row[:] for row in M]
    for sk, v_t in zip(sks, v):
        den = dot(sk, z) + eps
        for j in range(dv):
            r = 0.0
            for i in range(d):
                r += sk[i] * M[i][j]
            resid = v_t[j] - r / den
            for i in range(d):
                new_M[i][j] += sk[i] * resid
    new_z = z[:]
    for sk in sks:
        for i in range(d):
            new_z[i] += sk[i]
    return new_M, new_z


def layer_one_head(Q, K, V, beta, N, update, eps, scale):
    """The whole layer for one head: Q/K/V are lists of rows (length L).

    Linear rule: the retrieval is taken from the history closed form and the state is
    never used.  Delta rule: the state is carried with ``delta_step``.
    Returns (O rows, M, z).
    """
    L = len(Q)
    d = len(Q[0])
    dv = len(V[0])
    g = 1.0 / (1.0 + math.exp(-beta)) if beta >= 0 else math.exp(beta) / (1.0 + math.exp(beta))
    M = [[0.0] * dv for _ in range(d)]
    z = [0.0] * d
    out = []
    for lo in range(0, L, N):
        hi = min(lo + N, L)
        q, k, v = Q[lo:hi], K[lo:hi], V[lo:hi]
        a_dot = local_attention(q, k, v, scale)
        for i in range(hi - lo):
            if update == "linear":
                a_mem = retrieval_from_history(q[i], K[:lo], V[:lo], eps)
            else:
                sq = [sigma(x) for x in q[i]]
                den = dot(sq, z) + eps
                a_mem = [dot(sq, [M[r][c] for r in range(d)]) / den for c in range(dv)]
            out.append([g * a_mem[c] + (1.0 - g) * a_dot[i][c] for c in range(dv)])
        if update == "delta":
            M, z = delta_step(k, v, M, z, eps)
    if update == "linear":
        M, z = state_from_history(K, V, d, dv)
    return out, M, z


def layer_with_projections(X, W_qkv, W_o, beta, N, update, eps, scale, H, d):
    """The layer from its input: X is a list of rows (tokens) of d_model numbers for one
    batch element; W_qkv is a list of 3 H d rows of d_model weights, W_o a list of
    d_model rows of H d weights (row j of W_o: the weights output feature j gives to the
    concatenated head outputs).  Eq. 5: q_h[t][j] = sum_i X[t][i] W_qkv[h d + j][i] (k, v
    from the next two blocks of H d rows); the heads run with ``layer_one_head``; Eq. 11:
    O[t][f] = sum_h sum_j A_h[t][j] W_o[f][h d + j].  Returns the rows of O.
    """
    L = len(X)
    dm = len(X[0])
    heads_out = []
    for h in range(H):
        blocks = []
        for p in range(3):
            rows = []
            for t in range(L):
                row = []
                for j in range(d):
                    w = W_qkv[p * H * d + h * d + j]
                    acc = 0.0
                    for i in range(dm):
                        acc += X[t][i] * w[i]
                    row.append(acc)
                rows.append(row)
            blocks.append(rows)
        out, _, _ = layer_one_head(blocks[0], blocks[1], blocks[2], beta[h], N, update, eps, scale)
        heads_out.append(out)
    O = []
    for t in range(L):
        row = []
        for f in range(len(W_o)):
            acc = 0.0
            for h in range(H):
                for j in range(d):
                    acc += heads_out[h][t][j] * W_o[f][h * d + j]
            row.append(acc)
        O.append(row)
    return O
