"""GPU parity of the layer around the heads: the Q/K/V projection (Eq. 5), the output
projection (Eq. 11) and the whole layer X -> O, through the C-ABI, against the CPU
oracle on the same seeded inputs.

Tolerances: a projection alone is exact up to its one rounding to bf16 (float32
accumulation), so every element is within one bf16 rounding of the float64 product:
|gpu - ref| <= 2^-8 |ref| + 1e-6 max|ref|.  The whole layer uses the bf16 output
tolerance of the per-head tests (tests/gpu_util.py), against the oracle with Q, K, V and
A rounded to bf16 between the steps (the layer's storage precision).
"""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from oracle import infini_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16).contiguous()


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_rounded_product(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements off by more than one bf16 rounding, "
                           f"worst {float(np.abs(got - ref).max()):.3e}")


PROJ_CASES = [
    # name, B, H, d, d_model, L
    ("h2-d128-dm256-ragged", 2, 2, 128, 256, 3 * 256 + 77),
    ("h3-d64-dm96-ragged-features", 1, 3, 64, 96, 300),     # 3Hd = 576, K = 96 (3 stages)
    ("h1-d64-dm32-one-token", 1, 1, 64, 32, 1),
    ("h8-d128-dm1024", 1, 8, 128, 1024, 512),
]


@pytest.mark.parametrize("case", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_projections_match_oracle(case):
    gu.require_gpu()
    name, B, H, d, dm, L = case
    gu.note(f"[layer] projections {name}: B={B} H={H} d={d} d_model={dm} L={L}")
    w = wl.Workload(name, B, H, d, 64, L, "bf16", "linear", seed=21)
    X, w_qkv, w_o = wl.layer_inputs(w, dm)
    with binding.InfiniAttention(B, H, d, 64, beta=[0.0] * H) as layer:
        q, k, v = layer.project_qkv(_dev(X), _dev(w_qkv))
        A = wl.round_to_bf16(np.random.default_rng(5).standard_normal((B, H, L, d)).astype(np.float32))
        o = layer.project_out(_dev(A), _dev(w_o))
        torch.cuda.synchronize()
        Qr, Kr, Vr = orc.project_qkv(X, w_qkv, H, d)
        for got, ref, nm in ((q, Qr, "Q"), (k, Kr, "K"), (v, Vr, "V")):
            assert tuple(got.shape) == (B, H, L, d)
            _check_rounded_product(_host(got), ref, nm)
        assert tuple(o.shape) == (B, L, dm)
        _check_rounded_product(_host(o), orc.project_out(A, w_o), "O")


LAYER_CASES = [
    # name, B, H, d, d_model, N, L, update, window segments
    ("linear-h2-d128-ragged", 2, 2, 128, 256, 256, 3 * 256 + 77, "linear", 0),
    ("delta-h2-d128-ragged", 2, 2, 128, 256, 256, 3 * 256 + 77, "delta", 0),
    ("linear-windows-of-2", 1, 2, 128, 256, 128, 5 * 128 + 9, "linear", 2),
    ("delta-windows-of-1-d64", 1, 3, 64, 192, 96, 3 * 96 + 40, "delta", 1),
    ("linear-dm-not-hd", 1, 2, 64, 160, 128, 300, "linear", 0),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_matches_oracle(case):
    gu.require_gpu()
    name, B, H, d, dm, N, L, update, win = case
    gu.note(f"[layer] forward_layer {name}: B={B} H={H} d={d} d_model={dm} N={N} L={L} {update} window={win}")
    w = wl.Workload(name, B, H, d, N, L, "bf16", update, seed=31)
    X, w_qkv, w_o = wl.layer_inputs(w, dm)
    beta = wl.beta_for(w)
    with binding.InfiniAttention(B, H, d, N, update=update, beta=beta, max_window_segments=win) as layer:
        out = layer.forward_layer(_dev(X), _dev(w_qkv), _dev(w_o))
        M, z = layer.get_state()
        torch.cuda.synchronize()
        O_ref, M_ref, z_ref = orc.layer_forward(X, w_qkv, w_o, beta, N, H, d, update, eps=w.eps,
                                                bf16_between=True)
        tol = gu.tol_for("bf16")
        gu.check_output(_host(out), O_ref, tol, "O")
        gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, tol)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_layer_equals_the_three_calls(update):
    """forward_layer = project_qkv, forward_stream, project_out (the same kernels in the same
    order: bit-identical), also across windows and a second call carrying the state."""
    gu.require_gpu()
    B, H, d, dm, N, L = 2, 2, 128, 256, 128, 4 * 128 + 50
    gu.note(f"[layer] three calls vs forward_layer, {update}")
    w = wl.Workload("three", B, H, d, N, L, "bf16", update, seed=41)
    X, w_qkv, w_o = (_dev(a) for a in wl.layer_inputs(w, dm))
    beta = wl.beta_for(w)
    kw = dict(update=update, beta=beta, max_window_segments=2)
    with binding.InfiniAttention(B, H, d, N, **kw) as one, binding.InfiniAttention(B, H, d, N, **kw) as three:
        for _ in range(2):
            o1 = one.forward_layer(X, w_qkv, w_o)
            q, k, v = three.project_qkv(X, w_qkv)
            a = three.forward_stream(q, k, v)
            o3 = three.project_out(a, w_o)
            torch.cuda.synchronize()
            assert torch.equal(o1, o3)
        M1, z1 = one.get_state()
        M3, z3 = three.get_state()
        assert torch.equal(M1, M3) and torch.equal(z1, z3)


def test_layer_rejects_bad_arguments():
    gu.require_gpu()
    with binding.InfiniAttention(1, 2, 64, 64, beta=[0.0, 0.0]) as layer:
        x = torch.zeros((1, 10, 100), dtype=torch.bfloat16, device="cuda")   # d_model not a multiple of 32
        with pytest.raises(binding.InfiniAttnError):
            layer.forward_layer(x, torch.zeros((384, 100), dtype=torch.bfloat16, device="cuda"),
                                torch.zeros((100, 128), dtype=torch.bfloat16, device="cuda"))
    with binding.InfiniAttention(1, 2, 64, 64, io_dtype="f32", beta=[0.0, 0.0]) as layer:
        x = torch.zeros((1, 10, 128), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(binding.InfiniAttnError) as e:
            layer.forward_layer(x, torch.zeros((384, 128), dtype=torch.bfloat16, device="cuda"),
                                torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda"))
        assert e.value.status == binding.ERR_UNSUPPORTED


def test_full_size_layer_sampled_against_oracle():
    """The throughput shape (B=1, H=8, d=128, d_model=1024, N=2048, 32K tokens) in one
    forward_layer call: sampled tokens of segments 0 and 1 (which depend only on the first
    4096 tokens) against the oracle."""
    gu.require_gpu()
    w = wl.WORKLOADS[wl.THROUGHPUT_WORKLOAD]
    H, d, N = w.heads, w.head_dim, w.segment_len
    dm = H * d
    gu.note(f"[layer] full size: {w.name}, d_model={dm}")
    X, w_qkv, w_o = wl.layer_inputs(w, dm)
    beta = wl.beta_for(w)
    Xd, Wq, Wo = _dev(X), _dev(w_qkv), _dev(w_o)
    with binding.InfiniAttention(1, H, d, N, update=w.update, beta=beta) as layer:
        out = layer.forward_layer(Xd, Wq, Wo)
        torch.cuda.synchronize()
        n2 = 2 * N
        O_ref, _, _ = orc.layer_forward(X[:, :n2], w_qkv, w_o, beta, N, H, d, w.update, eps=w.eps,
                                        bf16_between=True)
        rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(N - 8, N + 8), np.arange(n2 - 8, n2),
                                         np.random.default_rng(3).integers(0, n2, 96)]))
        got = _host(out[:, rows])
        gu.check_output(got, O_ref[:, rows], gu.tol_for("bf16"), "O sampled")
