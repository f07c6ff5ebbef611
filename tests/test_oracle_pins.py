"""Pins of the CPU oracle against things other than itself (CPU only).

Every check here compares ``oracle.infini_oracle`` with a value fixed from outside it:
a library routine the special case reduces to (torch's causal SDPA, torch's ELU,
scipy's expit), a closed form (linearised attention over the history, the state as a
sum of outer products, the affine form of the delta step), an invariant the page
states (delta leaves an existing binding unchanged, z is the same under both rules,
the first segment reads an empty memory), brute force by scalar loops
(``oracle.brute``), or a figure the pages print (``tests/golden``).

Formulas: architecture summary of "Leave No Context Behind" (arXiv 2404.07143,
paper-graph-ui.vercel.app), section 3.4, Eq. 4 and Eq. 6-10.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import brute
from oracle import infini_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkv(rng, B, H, L, d, scale=1.0):
    s = scale / math.sqrt(d)
    return tuple(rng.standard_normal((B, H, L, d)) * s for _ in range(3))


# ---------------------------------------------------------------- sigma and sigmoid

def test_sigma_matches_torch_elu_plus_one(rng):
    x = np.concatenate([rng.standard_normal(1000) * 3, [0.0, -0.0, 1e-30, -1e-30, -50.0, 50.0]])
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    # torch forms expm1(x) + 1, which loses the tiny values to cancellation: compare absolutely
    np.testing.assert_allclose(orc.elu_plus_one(x), ref, rtol=0, atol=4e-16)


def test_sigma_special_values():
    assert orc.elu_plus_one(np.array([0.0]))[0] == 1.0
    assert orc.elu_plus_one(np.array([2.5]))[0] == 3.5
    assert orc.elu_plus_one(np.array([-np.inf]))[0] == 0.0
    assert orc.elu_plus_one(np.array([-1.0]))[0] == math.exp(-1.0)
    assert np.all(orc.elu_plus_one(np.linspace(-30, 30, 601)) > 0)


def test_sigmoid_matches_scipy_expit(rng):
    b = np.concatenate([rng.standard_normal(100) * 10, [0.0, -700.0, 700.0]])
    np.testing.assert_allclose(orc.sigmoid(b), scipy.special.expit(b), rtol=1e-14, atol=0)
    assert orc.sigmoid(np.array([-np.inf]))[0] == 0.0
    assert orc.sigmoid(np.array([np.inf]))[0] == 1.0
    assert orc.sigmoid(np.array([0.0]))[0] == 0.5


# ---------------------------------------------------------------- local attention (Eq. 6)

@pytest.mark.parametrize("n,d", [(1, 8), (7, 16), (33, 64), (64, 128)])
def test_local_attention_is_causal_sdpa(rng, n, d):
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True, scale=scale)[0].numpy()
    np.testing.assert_allclose(orc.local_causal_attention(q, k, v, scale), ref, rtol=1e-12, atol=1e-14)


def test_local_attention_single_token_returns_value(rng):
    q, k, v = (rng.standard_normal((1, 16)) for _ in range(3))
    assert np.array_equal(orc.local_causal_attention(q, k, v, 0.25), v)


def test_local_attention_equal_keys_gives_prefix_means(rng):
    n, d = 12, 8
    q = rng.standard_normal((n, d))
    k = np.tile(rng.standard_normal((1, d)), (n, 1))
    v = rng.standard_normal((n, d))
    prefix_means = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(orc.local_causal_attention(q, k, v, 0.3), prefix_means, rtol=1e-13, atol=1e-15)


def test_local_attention_brute_force(rng):
    n, d = 9, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    ref = np.array(brute.local_attention(q.tolist(), k.tolist(), v.tolist(), 0.7))
    np.testing.assert_allclose(orc.local_causal_attention(q, k, v, 0.7), ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- retrieval (Eq. 7) and linear state (Eq. 8)

def test_retrieval_is_linearised_attention_over_history(rng):
    """Linear rule: A_mem of segment s equals the history closed form, by brute force."""
    L, N, d = 20, 6, 4
    Q, K, V = _rand_qkv(rng, 1, 1, L, d, scale=2.0)
    _, _, _, A_mem, _ = orc.forward(Q, K, V, [0.3], N, "linear", eps=1e-6, return_parts=True)
    q, k, v = Q[0, 0].tolist(), K[0, 0].tolist(), V[0, 0].tolist()
    for i in range(L):
        lo = (i // N) * N
        ref = brute.retrieval_from_history(q[i], k[:lo], v[:lo], 1e-6)
        np.testing.assert_allclose(A_mem[0, 0, i], ref, rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_first_segment_reads_zero_memory(rng, update):
    Q, K, V = _rand_qkv(rng, 1, 2, 10, 8)
    beta = [0.7, -1.2]
    O, _, _, A_mem, A_dot = orc.forward(Q, K, V, beta, 10, update, return_parts=True)
    assert np.all(A_mem == 0.0)
    for h in range(2):
        g = scipy.special.expit(beta[h])
        np.testing.assert_allclose(O[0, h], (1 - g) * A_dot[0, h], rtol=1e-15, atol=0)


@pytest.mark.parametrize("N", [1, 3, 5, 17, 40])
def test_linear_state_is_sum_of_outer_products_for_any_segment_length(rng, N):
    L, d = 17, 5
    Q, K, V = _rand_qkv(rng, 1, 1, L, d, scale=3.0)
    _, M, z = orc.forward(Q, K, V, [0.0], N, "linear")
    M_ref, z_ref = brute.state_from_history(K[0, 0].tolist(), V[0, 0].tolist(), d, d)
    np.testing.assert_allclose(M[0, 0], M_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z[0, 0], z_ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_state_ignores_token_order_inside_a_segment(rng, update):
    """Both updates are segment-level: every token of a segment reads the same old state."""
    n, d = 16, 6
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    M0, z0 = rng.standard_normal((d, d)), np.abs(rng.standard_normal(d)) * 10 + 1
    perm = rng.permutation(n)
    a = orc.advance(k, v, M0, z0, update, 1e-6)
    b = orc.advance(k[perm], v[perm], M0, z0, update, 1e-6)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=0)


# ---------------------------------------------------------------- delta rule (Eq. 9)

def test_delta_leaves_an_existing_binding_unchanged(rng):
    """Invariant stated on the page: rewriting a pair the memory already returns exactly
    leaves M unchanged while z still grows by the key mass."""
    n, d = 8, 16
    key = rng.standard_normal(d)
    val = rng.standard_normal(d)
    k = np.tile(key, (n, 1))
    v = np.tile(val, (n, 1))
    # first write into the empty memory (retrieves 0 / eps = 0), then the same pair again
    M1, z1 = orc.memory_update_delta(k, v, np.zeros((d, d)), np.zeros(d), eps=1e-6)
    sk = orc.elu_plus_one(key)
    np.testing.assert_allclose(M1, n * np.outer(sk, val), rtol=1e-14, atol=0)
    M2, z2 = orc.memory_update_delta(k, v, M1, z1, eps=0.0)
    assert np.linalg.norm(M2 - M1) / np.linalg.norm(M1) <= 1e-12
    np.testing.assert_allclose(z2, z1 + n * sk, rtol=1e-14, atol=0)


def test_delta_equals_linear_on_first_segment_and_z_is_shared(rng):
    L, N, d = 24, 8, 6
    Q, K, V = _rand_qkv(rng, 1, 1, L, d, scale=2.0)
    _, M_lin1, z_lin1 = orc.forward(Q[..., :N, :], K[..., :N, :], V[..., :N, :], [0.0], N, "linear")
    _, M_del1, z_del1 = orc.forward(Q[..., :N, :], K[..., :N, :], V[..., :N, :], [0.0], N, "delta")
    np.testing.assert_allclose(M_del1, M_lin1, rtol=1e-12, atol=1e-14)
    _, M_lin, z_lin = orc.forward(Q, K, V, [0.0], N, "linear")
    _, M_del, z_del = orc.forward(Q, K, V, [0.0], N, "delta")
    np.testing.assert_array_equal(z_lin, z_del)
    assert np.linalg.norm(M_lin - M_del) > 1e-3 * np.linalg.norm(M_lin)


def test_delta_step_affine_form(rng):
    """Eq. 9 rearranged: M_s = (I - sigma(K)^T D sigma(K)) M_{s-1} + sigma(K)^T V with
    D = diag(1 / (sigma(K) z_{s-1} + eps)).  M is not symmetric, so a transposed operand
    anywhere in the oracle's retrieved value fails this."""
    n, d, dv = 11, 5, 7
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    M0 = rng.standard_normal((d, dv))
    z0 = np.abs(rng.standard_normal(d)) + 0.5
    eps = 0.25
    sk = np.array([[brute.sigma(x) for x in row] for row in k])
    D = np.diag(1.0 / (sk @ z0 + eps))
    ref = (np.eye(d) - sk.T @ D @ sk) @ M0 + sk.T @ v
    M1, _ = orc.memory_update_delta(k, v, M0, z0, eps)
    np.testing.assert_allclose(M1, ref, rtol=1e-12, atol=1e-12)


def test_delta_step_brute_force(rng):
    n, d = 5, 3
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    M0, z0 = rng.standard_normal((d, d)), np.abs(rng.standard_normal(d)) + 1
    M_ref, z_ref = brute.delta_step(k.tolist(), v.tolist(), M0.tolist(), z0.tolist(), 1e-3)
    M1, z1 = orc.memory_update_delta(k, v, M0, z0, 1e-3)
    np.testing.assert_allclose(M1, M_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(z1, z_ref, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- gate (Eq. 10)

@pytest.mark.parametrize("update", ["linear", "delta"])
def test_gate_limits(rng, update):
    L, N, d = 30, 8, 8
    Q, K, V = _rand_qkv(rng, 1, 3, L, d)
    beta = [-np.inf, 0.0, np.inf]
    O, _, _, A_mem, A_dot = orc.forward(Q, K, V, beta, N, update, return_parts=True)
    # beta -> -inf: plain causal softmax attention per segment (invariant 1)
    for lo, hi in orc.segment_bounds(L, N):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[0, 0, lo:hi])[None], torch.from_numpy(K[0, 0, lo:hi])[None],
            torch.from_numpy(V[0, 0, lo:hi])[None], is_causal=True)[0].numpy()
        np.testing.assert_allclose(O[0, 0, lo:hi], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O[0, 1], 0.5 * (A_mem[0, 1] + A_dot[0, 1]), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(O[0, 2], A_mem[0, 2])


# ---------------------------------------------------------------- whole layer

@pytest.mark.parametrize("update", ["linear", "delta"])
def test_layer_matches_scalar_loops(rng, update):
    B, H, L, N, d = 1, 2, 13, 4, 3      # ragged last segment (1 token)
    Q, K, V = _rand_qkv(rng, B, H, L, d, scale=2.0)
    beta = [0.4, -0.9]
    O, M, z = orc.forward(Q, K, V, beta, N, update, eps=1e-6)
    for h in range(H):
        o_ref, M_ref, z_ref = brute.layer_one_head(
            Q[0, h].tolist(), K[0, h].tolist(), V[0, h].tolist(), beta[h], N, update, 1e-6, 1 / math.sqrt(d))
        np.testing.assert_allclose(O[0, h], o_ref, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(M[0, h], M_ref, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(z[0, h], z_ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_heads_and_batch_are_independent(rng, update):
    B, H, L, N, d = 2, 3, 20, 8, 4
    Q, K, V = _rand_qkv(rng, B, H, L, d)
    beta = np.array([0.1, -0.5, 1.5])
    O, M, z = orc.forward(Q, K, V, beta, N, update)
    perm = np.array([2, 0, 1])
    O2, M2, z2 = orc.forward(Q[:, perm], K[:, perm], V[:, perm], beta[perm], N, update)
    np.testing.assert_array_equal(O2, O[:, perm])
    np.testing.assert_array_equal(M2, M[:, perm])
    O3, _, _ = orc.forward(Q[::-1], K[::-1], V[::-1], beta, N, update)
    np.testing.assert_array_equal(O3, O[::-1])


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_output_is_linear_in_values(rng, update):
    """For fixed Q, K and a zero start, O and M are linear in V under both rules
    (Eq. 9 is affine in M_{s-1} with a K-only coefficient)."""
    L, N, d = 24, 8, 5
    Q, K, V1 = _rand_qkv(rng, 1, 1, L, d)
    V2 = rng.standard_normal(V1.shape)
    O1, M1, _ = orc.forward(Q, K, V1, [0.2], N, update)
    O2, M2, _ = orc.forward(Q, K, V2, [0.2], N, update)
    O3, M3, _ = orc.forward(Q, K, V1 - 2.5 * V2, [0.2], N, update)
    np.testing.assert_allclose(O3, O1 - 2.5 * O2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(M3, M1 - 2.5 * M2, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_splitting_the_stream_at_a_segment_boundary_changes_nothing(rng, update):
    L, N, d = 40, 8, 6
    Q, K, V = _rand_qkv(rng, 1, 2, L, d)
    beta = [0.3, -0.3]
    O, M, z = orc.forward(Q, K, V, beta, N, update)
    cut = 24
    Oa, Ma, za = orc.forward(Q[..., :cut, :], K[..., :cut, :], V[..., :cut, :], beta, N, update)
    Ob, Mb, zb = orc.forward(Q[..., cut:, :], K[..., cut:, :], V[..., cut:, :], beta, N, update,
                             M0=Ma, z0=za)
    np.testing.assert_array_equal(np.concatenate([Oa, Ob], axis=2), O)
    np.testing.assert_array_equal(Mb, M)
    np.testing.assert_array_equal(zb, z)


def test_softmax_scale_is_an_explicit_parameter(rng):
    Q, K, V = _rand_qkv(rng, 1, 1, 16, 8, scale=4.0)
    O_default, _, _ = orc.forward(Q, K, V, [-np.inf], 16)
    O_explicit, _, _ = orc.forward(Q, K, V, [-np.inf], 16, scale=1 / math.sqrt(8))
    O_dmodel, _, _ = orc.forward(Q, K, V, [-np.inf], 16, scale=1 / math.sqrt(8 * 8))
    np.testing.assert_array_equal(O_default, O_explicit)
    assert not np.allclose(O_default, O_dmodel)


# ---------------------------------------------------------------- figures printed on the pages

def test_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        g = json.load(f)
    fp = g["memory_footprint_per_layer"]
    m_numbers, z_numbers = orc.state_numbers_per_layer(fp["heads"], fp["d_key"], fp["d_value"])
    assert m_numbers == fp["M_numbers"] and z_numbers == fp["z_numbers"]
    assert abs((m_numbers + z_numbers) * 4 / 2**20 - fp["approx_MB_float32"]) < 0.01
    u = g["training_unroll"]
    assert len(orc.segment_bounds(u["tokens"], u["segment_len"])) == u["segments"]
    bk = g["booksum_segments"]
    bounds = orc.segment_bounds(bk["tokens"], bk["segment_len"])
    full = [b for b in bounds if b[1] - b[0] == bk["segment_len"]]
    assert len(full) == bk["full_segments"]
    assert (bounds[-1][1] - bounds[-1][0] < bk["segment_len"]) == bk["final_segment_shorter"]


# ---------------------------------------------------------------- separate local Q/K
# The summary page's training notes apply position embeddings to the local arm's Q and K
# only, after the memory read and update ("Compressive Memory" / "Training Infrastructure"
# subsections); the oracle takes those as optional inputs.

def _pe_inputs(rng, B=1, H=2, L=70, d=16):
    from tests.rope import rope
    Q, K, V = (rng.standard_normal((B, H, L, d)) / math.sqrt(d) for _ in range(3))
    return Q, K, V, rope(Q), rope(K)


def test_local_qk_with_gate_off_is_causal_sdpa_of_the_local_inputs(rng):
    Q, K, V, Ql, Kl = _pe_inputs(rng)
    N = 32
    O, _, _ = orc.forward(Q, K, V, np.full(2, -np.inf), N, "linear", Q_local=Ql, K_local=Kl)
    for lo in range(0, Q.shape[2], N):
        hi = min(lo + N, Q.shape[2])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Ql[..., lo:hi, :]), torch.from_numpy(Kl[..., lo:hi, :]),
            torch.from_numpy(V[..., lo:hi, :]), is_causal=True, scale=1.0 / math.sqrt(Q.shape[-1])).numpy()
        np.testing.assert_allclose(O[..., lo:hi, :], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_local_qk_leave_the_memory_path_unchanged(rng, update):
    Q, K, V, Ql, Kl = _pe_inputs(rng)
    beta = rng.standard_normal(2)
    base = orc.forward(Q, K, V, beta, 24, update, return_parts=True)
    pe = orc.forward(Q, K, V, beta, 24, update, return_parts=True, Q_local=Ql, K_local=Kl)
    for i in (1, 2, 3):   # M, z and A_mem do not see the local inputs
        assert np.array_equal(base[i], pe[i])
    assert not np.allclose(base[4], pe[4])   # A_dot does
    same = orc.forward(Q, K, V, beta, 24, update, return_parts=True, Q_local=Q, K_local=K)
    for x, y in zip(base, same):
        assert np.array_equal(x, y)


def test_rope_is_a_rotation_and_shifts_scores_by_relative_position(rng):
    """Pins the test helper itself: norms are kept, and q.k after RoPE depends only on the
    position difference."""
    from tests.rope import rope
    d = 8
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    for p in (0, 3, 11):
        np.testing.assert_allclose(np.linalg.norm(rope(q, pos0=p)), np.linalg.norm(q), rtol=1e-14)
    s1 = rope(q, pos0=7) @ rope(k, pos0=4).T
    s2 = rope(q, pos0=13) @ rope(k, pos0=10).T
    np.testing.assert_allclose(s1, s2, rtol=1e-12)


# ---------------------------------------------------------------- the projections (Eq. 5, Eq. 11)
# Section "Standard Dot-Product Attention" (Query, Key, Value projections) and section
# "Multi-Head Infini-Attention": each head has its own W_Q, W_K, W_V (d_model x d); the
# head outputs are concatenated in order and multiplied by W_O (H d x d_model).  Weights
# here are in the "out x in" layout the oracle takes.

def test_round_to_bf16_matches_torch_and_ties_go_to_even(rng):
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_to_bf16(x.astype(np.float64)), ref)
    # ties: bf16 spacing at 1 is 2^-7
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -9])
    np.testing.assert_array_equal(orc.round_to_bf16(ties), [1.0, 1 + 2.0 ** -6, -1.0, 3 * 2.0 ** -9])
    assert orc.round_to_bf16(np.array([0.0]))[0] == 0.0


def _layer_weights(rng, H, d, dm, scale=1.0):
    w_qkv = rng.standard_normal((3 * H * d, dm)) * (scale / math.sqrt(dm))
    w_o = rng.standard_normal((dm, H * d)) / math.sqrt(H * d)
    return w_qkv, w_o


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_layer_with_projections_matches_scalar_loops(rng, update):
    B, H, d, dm, L, N = 2, 2, 3, 5, 9, 4   # ragged last segment
    X = rng.standard_normal((B, L, dm))
    w_qkv, w_o = _layer_weights(rng, H, d, dm, scale=1.5)
    beta = [0.7, -0.4]
    O, _, _ = orc.layer_forward(X, w_qkv, w_o, beta, N, H, d, update)
    assert O.shape == (B, L, dm)
    for b in range(B):
        ref = brute.layer_with_projections(X[b].tolist(), w_qkv.tolist(), w_o.tolist(), beta, N, update,
                                           1e-6, 1 / math.sqrt(d), H, d)
        np.testing.assert_allclose(O[b], ref, rtol=1e-10, atol=1e-13)


def test_output_projection_is_a_sum_of_per_head_blocks(rng):
    """[A_1; ...; A_H] W_O = sum_h A_h W_O[h d:(h+1) d, :] (block form of the concatenation)."""
    B, H, L, d, dm = 2, 3, 7, 4, 6
    A = rng.standard_normal((B, H, L, d))
    W_O = rng.standard_normal((H * d, dm))   # the page's orientation
    ref = sum(A[:, h] @ W_O[h * d:(h + 1) * d] for h in range(H))
    np.testing.assert_allclose(orc.project_out(A, W_O.T), ref, rtol=1e-12, atol=1e-13)


def test_qkv_projection_per_head_columns(rng):
    """Q_h = X W_Q^(h) with W_Q^(h) the d columns of head h, and K, V from their own blocks."""
    B, L, H, d, dm = 2, 5, 3, 4, 7
    X = rng.standard_normal((B, L, dm))
    W = [[rng.standard_normal((dm, d)) for _ in range(H)] for _ in range(3)]   # [part][head]: dm x d
    w_qkv = np.concatenate([W[p][h].T for p in range(3) for h in range(H)], axis=0)
    Q, K, V = orc.project_qkv(X, w_qkv, H, d)
    for p, got in enumerate((Q, K, V)):
        for h in range(H):
            np.testing.assert_allclose(got[:, h], X @ W[p][h], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_layer_identity_projections_reduce_to_the_heads(rng, update):
    """d_model = H d, W_Q = W_K = W_V = W_O = I: O is the per-head layer on X cut into heads."""
    B, H, d, L, N = 1, 2, 4, 11, 4
    dm = H * d
    X = rng.standard_normal((B, L, dm)) / math.sqrt(d)
    eye = np.eye(dm)
    beta = [0.3, -1.1]
    O, M, z = orc.layer_forward(X, np.concatenate([eye, eye, eye]), eye, beta, N, H, d, update)
    Xh = X.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    A, M2, z2 = orc.forward(Xh, Xh, Xh, beta, N, update)
    np.testing.assert_allclose(O, A.transpose(0, 2, 1, 3).reshape(B, L, dm), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M, M2, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_layer_relabelling_heads_changes_nothing(rng, update):
    """Permuting the heads in W_qkv, W_O and beta together leaves O unchanged."""
    H, d, dm, L, N = 3, 4, 10, 12, 5
    X = rng.standard_normal((1, L, dm))
    w_qkv, w_o = _layer_weights(rng, H, d, dm)
    beta = np.array([0.5, -0.3, 1.2])
    O, _, _ = orc.layer_forward(X, w_qkv, w_o, beta, N, H, d, update)
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(p * H * d + h * d, p * H * d + (h + 1) * d) for p in range(3) for h in perm])
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in perm])
    O2, _, _ = orc.layer_forward(X, w_qkv[rows], w_o[:, cols], beta[perm], N, H, d, update)
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-13)


def test_layer_is_linear_in_the_output_weights(rng):
    H, d, dm, L, N = 2, 4, 8, 10, 4
    X = rng.standard_normal((2, L, dm))
    w_qkv, w1 = _layer_weights(rng, H, d, dm)
    w2 = rng.standard_normal(w1.shape)
    O1, _, _ = orc.layer_forward(X, w_qkv, w1, [0.1, 0.2], N, H, d)
    O2, _, _ = orc.layer_forward(X, w_qkv, w2, [0.1, 0.2], N, H, d)
    O3, _, _ = orc.layer_forward(X, w_qkv, w1 - 3 * w2, [0.1, 0.2], N, H, d)
    np.testing.assert_allclose(O3, O1 - 3 * O2, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- incremental decoding
# Tokens fed one at a time (the summary's "fast streaming inference"): a per-token softmax
# over the segment's cache and a memory written when the segment closes must give the
# segment formulation's outputs and states exactly (causality inside the segment).

@pytest.mark.parametrize("update", ["linear", "delta"])
def test_token_by_token_decoding_equals_the_segment_forward(rng, update):
    B, H, L, N, d = 2, 2, 23, 8, 5   # two closed segments and a partial one
    Q, K, V = _rand_qkv(rng, B, H, L, d, scale=1.5)
    beta = [0.6, -0.8]
    O, M, z = orc.forward(Q, K, V, beta, N, update)
    O2, M2, z2, open_tokens = orc.decode_stream(Q, K, V, beta, N, update)
    assert open_tokens == 0
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(M2, M, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(z2, z, rtol=1e-13, atol=0)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_decoding_leaves_an_open_segment_out_of_the_memory(rng, update):
    B, H, L, N, d = 1, 2, 19, 8, 4
    Q, K, V = _rand_qkv(rng, B, H, L, d)
    beta = [0.2, 0.9]
    _, M, z, open_tokens = orc.decode_stream(Q, K, V, beta, N, update, flush=False)
    assert open_tokens == L % N
    _, M_ref, z_ref = orc.forward(Q[:, :, :16], K[:, :, :16], V[:, :, :16], beta, N, update)
    np.testing.assert_allclose(M, M_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(z, z_ref, rtol=1e-13, atol=0)
