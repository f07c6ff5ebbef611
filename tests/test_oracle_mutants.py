"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (on the CPU, by swapping one of its
functions for a wrong version) and checks that at least one of the pins in
``test_oracle_pins`` then fails.  Nothing here touches the GPU library.
"""

import numpy as np
import pytest

from oracle import infini_oracle as orc
from tests import test_oracle_pins as pins


def _retrieval_transposed(q, M, z, eps):
    sq = orc.elu_plus_one(q)
    return (sq @ np.asarray(M).T) / (sq @ z + eps)[:, None]


def _retrieval_no_z(q, M, z, eps):
    sq = orc.elu_plus_one(q)
    return (sq @ M) / (sq.sum(axis=1) + eps)[:, None]


def _delta_wrong_sign(k, v, M, z, eps):
    sk = orc.elu_plus_one(k)
    r = (sk @ M) / (sk @ z + eps)[:, None]
    return M + sk.T @ (v + r), z + sk.sum(axis=0)


def _delta_reads_new_z(k, v, M, z, eps):
    sk = orc.elu_plus_one(k)
    z_new = z + sk.sum(axis=0)
    r = (sk @ M) / (sk @ z_new + eps)[:, None]
    return M + sk.T @ (v - r), z_new


def _delta_transposed(k, v, M, z, eps):
    sk = orc.elu_plus_one(k)
    r = (sk @ np.asarray(M).T) / (sk @ z + eps)[:, None]
    return M + sk.T @ (v - r), z + sk.sum(axis=0)


def _linear_forgets_z(k, v, M, z):
    sk = orc.elu_plus_one(k)
    return M + sk.T @ v, np.asarray(z, dtype=np.float64)


def _linear_raw_keys(k, v, M, z):
    k = np.asarray(k, dtype=np.float64)
    return M + k.T @ v, z + orc.elu_plus_one(k).sum(axis=0)


def _attention_off_by_one(q, k, v, scale):
    n = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(np.triu(np.ones((n, n), dtype=bool), k=2), -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


def _attention_unscaled(q, k, v, scale):
    return orc.__dict__["_orig_attention"](q, k, v, 1.0)


def _gate_swapped(a_mem, a_dot, beta):
    g = float(orc.sigmoid(np.array([beta]))[0])
    return g * np.asarray(a_dot) + (1.0 - g) * np.asarray(a_mem)


def _segment_ignores_local_qk(q, k, v, M, z, beta, update, eps, scale, q_local=None, k_local=None):
    return orc.__dict__["_orig_segment_forward"](q, k, v, M, z, beta, update, eps, scale)


def _segment_local_qk_in_memory(q, k, v, M, z, beta, update, eps, scale, q_local=None, k_local=None):
    ql = q if q_local is None else q_local
    kl = k if k_local is None else k_local
    return orc.__dict__["_orig_segment_forward"](ql, kl, v, M, z, beta, update, eps, scale)


def _project_out_feature_major(A, W_o):
    A = np.asarray(A, dtype=np.float64)
    B, H, L, d = A.shape
    cat = A.transpose(0, 2, 3, 1).reshape(B, L, H * d)   # heads interleaved, not concatenated
    return cat @ np.asarray(W_o, dtype=np.float64).T


def _project_out_untransposed(A, W_o):
    A = np.asarray(A, dtype=np.float64)
    B, H, L, d = A.shape
    return A.transpose(0, 2, 1, 3).reshape(B, L, H * d) @ np.asarray(W_o, dtype=np.float64)


def _project_qkv_k_v_swapped(X, W_qkv, heads, head_dim):
    q, k, v = orc.__dict__["_orig_project_qkv"](X, W_qkv, heads, head_dim)
    return q, v, k


def _project_qkv_head_interleaved(X, W_qkv, heads, head_dim):
    X = np.asarray(X, dtype=np.float64)
    Y = X @ np.asarray(W_qkv, dtype=np.float64).T
    B, L, _ = X.shape
    H, d = heads, head_dim
    return tuple(Y[:, :, p * H * d:(p + 1) * H * d].reshape(B, L, d, H).transpose(0, 3, 1, 2) for p in range(3))


def _round_truncates(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _decode_excludes_current_token(q, k, v, cache_k, cache_v, M, z, beta, eps, scale):
    a, ck, cv = orc.__dict__["_orig_decode_token"](q, k, v, cache_k, cache_v, M, z, beta, eps, scale)
    if np.asarray(cache_k).size == 0:
        return a, ck, cv
    a2, _, _ = orc.__dict__["_orig_decode_token"](q, np.asarray(cache_k)[-1], np.asarray(cache_v)[-1],
                                                   np.asarray(cache_k)[:-1], np.asarray(cache_v)[:-1],
                                                   M, z, beta, eps, scale)
    return a2, ck, cv


def _decode_unscaled(q, k, v, cache_k, cache_v, M, z, beta, eps, scale):
    return orc.__dict__["_orig_decode_token"](q, k, v, cache_k, cache_v, M, z, beta, eps, 1.0)


def _elu_without_one(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0.0)))


MUTANTS = {
    "retrieval-transposed-M": ("memory_retrieval", _retrieval_transposed),
    "retrieval-drops-z": ("memory_retrieval", _retrieval_no_z),
    "delta-wrong-sign": ("memory_update_delta", _delta_wrong_sign),
    "delta-reads-updated-z": ("memory_update_delta", _delta_reads_new_z),
    "delta-transposed-M": ("memory_update_delta", _delta_transposed),
    "linear-forgets-z": ("memory_update_linear", _linear_forgets_z),
    "linear-binds-raw-keys": ("memory_update_linear", _linear_raw_keys),
    "attention-mask-off-by-one": ("local_causal_attention", _attention_off_by_one),
    "attention-unscaled": ("local_causal_attention", _attention_unscaled),
    "gate-swapped": ("gate", _gate_swapped),
    "elu-without-plus-one": ("elu_plus_one", _elu_without_one),
    "local-qk-ignored": ("segment_forward", _segment_ignores_local_qk),
    "local-qk-fed-to-memory": ("segment_forward", _segment_local_qk_in_memory),
    "out-projection-heads-interleaved": ("project_out", _project_out_feature_major),
    "out-projection-untransposed": ("project_out", _project_out_untransposed),
    "qkv-projection-k-v-swapped": ("project_qkv", _project_qkv_k_v_swapped),
    "qkv-projection-heads-interleaved": ("project_qkv", _project_qkv_head_interleaved),
    "bf16-rounding-truncates": ("round_to_bf16", _round_truncates),
    "decode-excludes-current-token": ("decode_token", _decode_excludes_current_token),
    "decode-unscaled-scores": ("decode_token", _decode_unscaled),
}


def _all_pins(rng):
    """Every pin, called directly (each raises AssertionError on a mismatch)."""
    yield lambda: pins.test_sigma_matches_torch_elu_plus_one(rng)
    yield lambda: pins.test_local_attention_is_causal_sdpa(rng, 33, 64)
    yield lambda: pins.test_local_attention_brute_force(rng)
    yield lambda: pins.test_retrieval_is_linearised_attention_over_history(rng)
    for u in ("linear", "delta"):
        yield lambda u=u: pins.test_first_segment_reads_zero_memory(rng, u)
        yield lambda u=u: pins.test_gate_limits(rng, u)
        yield lambda u=u: pins.test_layer_matches_scalar_loops(rng, u)
    yield lambda: pins.test_linear_state_is_sum_of_outer_products_for_any_segment_length(rng, 5)
    yield lambda: pins.test_delta_leaves_an_existing_binding_unchanged(rng)
    yield lambda: pins.test_delta_equals_linear_on_first_segment_and_z_is_shared(rng)
    yield lambda: pins.test_delta_step_affine_form(rng)
    yield lambda: pins.test_delta_step_brute_force(rng)
    yield lambda: pins.test_local_qk_with_gate_off_is_causal_sdpa_of_the_local_inputs(rng)
    for u in ("linear", "delta"):
        yield lambda u=u: pins.test_local_qk_leave_the_memory_path_unchanged(rng, u)
    yield lambda: pins.test_round_to_bf16_matches_torch_and_ties_go_to_even(rng)
    yield lambda: pins.test_output_projection_is_a_sum_of_per_head_blocks(rng)
    yield lambda: pins.test_qkv_projection_per_head_columns(rng)
    for u in ("linear", "delta"):
        yield lambda u=u: pins.test_layer_with_projections_matches_scalar_loops(rng, u)
        yield lambda u=u: pins.test_token_by_token_decoding_equals_the_segment_forward(rng, u)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_a_planted_mistake_fails_a_pin(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(orc.__dict__, "_orig_attention", orc.local_causal_attention)
    monkeypatch.setitem(orc.__dict__, "_orig_segment_forward", orc.segment_forward)
    monkeypatch.setitem(orc.__dict__, "_orig_project_qkv", orc.project_qkv)
    monkeypatch.setitem(orc.__dict__, "_orig_decode_token", orc.decode_token)
    monkeypatch.setattr(orc, attr, fn)
    rng = np.random.default_rng(99)
    caught = []
    for pin in _all_pins(rng):
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake {name!r}"
