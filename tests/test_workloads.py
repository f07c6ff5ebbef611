"""The seeded input generator (CPU only): deterministic, bf16-exact, per-segment."""

import math

import numpy as np
import pytest

from compressive_memory_transformer_segment_amd import workloads as wl


def test_round_to_bf16_ties_to_even_and_exactness():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0, 3.0e38], dtype=np.float32)
    r = wl.round_to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert r[1] == 1.0
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert r[2] == np.float32(1.0 + 2**-6)
    assert r[3] == 1.0
    assert r[4] == -2.5 and r[5] == 0.0
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
def test_workload_shapes_and_determinism(name):
    w = wl.WORKLOADS[name]
    q, k, v = wl.segment_inputs(w, 0, 0)
    assert q.shape == (w.heads, min(w.segment_len, w.n_tokens), w.head_dim)
    q2, _, _ = wl.segment_inputs(w, 0, 0)
    assert np.array_equal(q, q2)
    if w.io_dtype == "bf16":
        for x in (q, k, v):
            assert np.all((x.view(np.uint32) & 0xFFFF) == 0)
    std = float(v.std())
    expect = 1.0 / math.sqrt(w.head_dim)
    lo, hi = (0.6, 1.6) if w.token_scale else (0.95, 1.05)
    assert lo * expect < std < hi * expect


def test_stream_is_concatenation_of_segments():
    w = wl.WORKLOADS["h8-d128-n2048-l32k-linear"].with_tokens(2048 * 2 + 100)
    Q, K, V = wl.stream_inputs(w)
    assert Q.shape == (1, 8, 4196, 128)
    q, k, v = wl.segment_inputs(w, 0, 2)
    assert q.shape[1] == 100
    assert np.array_equal(K[0, :, 4096:], k)


def test_planted_pair():
    w = wl.WORKLOADS["h8-d128-n2048-l1m-linear-planted"].with_tokens(3 * 2048)
    k_star, v_star = wl.planted_pair(w)
    assert abs(float(np.linalg.norm(k_star.astype(np.float64))) - 1.0) < 1e-2
    _, k0, v0 = wl.segment_inputs(w, 0, 0)
    assert np.array_equal(k0[:, 0], np.broadcast_to(k_star, k0[:, 0].shape))
    assert np.array_equal(v0[:, 0], np.broadcast_to(v_star, v0[:, 0].shape))
    q_last, _, _ = wl.segment_inputs(w, 0, 2)
    assert np.array_equal(q_last[:, -1], np.broadcast_to(k_star, q_last[:, -1].shape))
    q_mid, _, _ = wl.segment_inputs(w, 0, 1)
    assert not np.array_equal(q_mid[:, -1], np.broadcast_to(k_star, q_mid[:, -1].shape))


def test_beta_draws():
    assert np.all(wl.beta_for(wl.WORKLOADS["tiny-f32-h1-d64-n64-l256-linear"]) == 0)
    b = wl.beta_for(wl.WORKLOADS["h8-d128-n2048-l32k-linear"])
    assert b.shape == (8,) and np.all(np.isfinite(b)) and np.std(b) > 0.1
