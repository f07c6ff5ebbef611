"""GPU parity: the HIP library through its C-ABI against the CPU oracle, element by
element, at sizes the oracle finishes in seconds (several tiles, ragged tails, edge
cases).  Tolerances are in tests/gpu_util.py."""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from oracle import infini_oracle as orc
from tests import gpu_util as gu
from tests.rope import rope

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, d, N, L, dtype, update
    ("bf16-linear-d128-ragged", 2, 3, 128, 256, 3 * 256 + 77, "bf16", "linear"),
    ("bf16-delta-d128-ragged", 2, 3, 128, 256, 3 * 256 + 77, "bf16", "delta"),
    ("bf16-linear-d64", 1, 2, 64, 192, 2 * 192 + 1, "bf16", "linear"),
    ("bf16-delta-d64", 1, 2, 64, 192, 4 * 192, "bf16", "delta"),
    ("bf16-linear-n100", 1, 2, 128, 100, 250, "bf16", "linear"),
    ("bf16-delta-n100", 1, 2, 128, 100, 250, "bf16", "delta"),
    ("bf16-linear-n1", 1, 2, 128, 1, 5, "bf16", "linear"),
    ("bf16-delta-n1", 1, 2, 64, 1, 4, "bf16", "delta"),
    ("bf16-linear-one-partial-segment", 1, 2, 128, 2048, 300, "bf16", "linear"),
    ("bf16-linear-one-token", 1, 1, 128, 2048, 1, "bf16", "linear"),
    ("bf16-delta-n2048-3seg", 1, 2, 128, 2048, 2 * 2048 + 1000, "bf16", "delta"),
    # segments longer than the 2K of the pages' runs: 16 query tiles, 64 key tiles on the diagonal
    ("bf16-linear-n4096-ragged", 1, 1, 128, 4096, 4096 + 1333, "bf16", "linear"),
    ("bf16-delta-n4096-ragged", 1, 1, 128, 4096, 4096 + 1333, "bf16", "delta"),
    # enough (batch, head) pairs for the delta chain's 16-rows-per-workgroup form
    ("bf16-delta-d128-b4h8-wide-chain", 4, 8, 128, 128, 3 * 128 + 50, "bf16", "delta"),
    ("bf16-delta-d64-b8h8-wide-chain", 8, 8, 64, 64, 4 * 64 + 5, "bf16", "delta"),
    ("f32-linear-d128", 1, 2, 128, 96, 3 * 96 + 5, "f32", "linear"),
    ("f32-delta-d128", 1, 2, 128, 96, 3 * 96 + 5, "f32", "delta"),
    ("f32-delta-d64", 2, 1, 64, 64, 200, "f32", "delta"),
]


def _run_case(w, beta, Q, K, V, want_parts=True, **layer_kw):
    dev = [gu.to_dev(x, w.io_dtype) for x in (Q, K, V)]
    with binding.InfiniAttention(w.batch, w.heads, w.head_dim, w.segment_len, update=w.update,
                                 io_dtype=w.io_dtype, eps=w.eps, beta=beta, **layer_kw) as layer:
        a_mem = torch.empty(dev[0].shape, dtype=torch.float32, device="cuda") if want_parts else None
        a_dot = torch.empty(dev[0].shape, dtype=torch.float32, device="cuda") if want_parts else None
        out = layer.forward_stream(*dev, a_mem=a_mem, a_dot=a_dot)
        M, z = layer.get_state()
        torch.cuda.synchronize()
        res = dict(out=out.float().cpu().numpy(), M=M.cpu().numpy(), z=z.cpu().numpy())
        if want_parts:
            res["a_mem"] = a_mem.cpu().numpy()
            res["a_dot"] = a_dot.cpu().numpy()
        return res


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_matches_oracle(case):
    gu.require_gpu()
    name, B, H, d, N, L, dtype, update = case
    w = wl.Workload(name, B, H, d, N, L, dtype, update, seed=11)
    gu.note(f"[parity] {name}: B={B} H={H} d={d} N={N} L={L} {dtype} {update} via forward_stream_ex")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    res = _run_case(w, beta, Q, K, V)
    O_ref, M_ref, z_ref, A_mem_ref, A_dot_ref = orc.forward(Q, K, V, beta, N, update, eps=w.eps,
                                                            return_parts=True)
    tol = gu.tol_for(dtype)
    gu.check_output(res["out"], O_ref, tol)
    gu.check_part(res["a_dot"], A_dot_ref, tol, "A_dot")
    for lo, hi in orc.segment_bounds(L, N):
        gu.check_part(res["a_mem"][:, :, lo:hi], A_mem_ref[:, :, lo:hi], tol, f"A_mem[{lo}:{hi}]")
    gu.check_state(res["M"], res["z"], M_ref, z_ref, tol)


def test_tiny_f32_workload_exactly_as_specified():
    """One head, d=64, N=64, L=256, fp32 I/O, linear rule, beta = 0, eps = 1e-6, seed 0."""
    gu.require_gpu()
    w = wl.WORKLOADS["tiny-f32-h1-d64-n64-l256-linear"]
    gu.note(f"[parity] {w.name}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    res = _run_case(w, beta, Q, K, V)
    O_ref, M_ref, z_ref, A_mem_ref, A_dot_ref = orc.forward(Q, K, V, beta, w.segment_len, w.update,
                                                            eps=w.eps, return_parts=True)
    tol = gu.F32_TOL
    gu.check_output(res["out"], O_ref, tol)
    gu.check_part(res["a_mem"], A_mem_ref, tol, "A_mem")
    gu.check_state(res["M"], res["z"], M_ref, z_ref, tol)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_gate_limits_on_gpu(update):
    """beta = -inf gives causal softmax attention per segment; beta = +inf gives A_mem."""
    gu.require_gpu()
    w = wl.Workload(f"gate-{update}", 1, 2, 128, 256, 700, "bf16", update, seed=5)
    gu.note(f"[parity] gate limits {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = np.array([-np.inf, np.inf], dtype=np.float32)
    res = _run_case(w, beta, Q, K, V)
    O_ref, _, _, A_mem_ref, A_dot_ref = orc.forward(Q, K, V, beta, 256, update, eps=w.eps, return_parts=True)
    gu.check_output(res["out"][:, 0], A_dot_ref[:, 0], gu.BF16_TOL, "beta=-inf")
    gu.check_output(res["out"][:, 1], O_ref[:, 1], gu.BF16_TOL, "beta=+inf")
    # +inf: the output is exactly the bf16 rounding of the kernel's own A_mem
    am = torch.from_numpy(res["a_mem"][:, 1]).to(torch.bfloat16).float().numpy()
    assert np.array_equal(res["out"][:, 1], am)
    # first segment reads an empty memory: A_mem = 0 exactly
    assert np.all(res["a_mem"][:, :, :256] == 0)


@pytest.mark.parametrize("update,B,H,N,S", [("linear", 1, 4, 512, 4), ("delta", 1, 4, 512, 4),
                                            ("linear", 4, 8, 1024, 4), ("delta", 4, 8, 1024, 4)])
def test_results_are_deterministic(update, B, H, N, S):
    """Bit-identical reruns.  The batch-4 cases run one state-pass workgroup per compute unit
    with two chunks per segment, where every workgroup reads the key sums of the segments
    before its own while others are still running."""
    gu.require_gpu()
    w = wl.Workload(f"det-{update}-b{B}", B, H, 128, N, S * N, "bf16", update, seed=8)
    gu.note(f"[parity] determinism {w.name}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    r1 = _run_case(w, beta, Q, K, V, want_parts=False)
    for _ in range(2):
        r2 = _run_case(w, beta, Q, K, V, want_parts=False)
        assert np.array_equal(r1["out"], r2["out"])
        assert np.array_equal(r1["M"], r2["M"]) and np.array_equal(r1["z"], r2["z"])


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_segment_calls_and_windows_match_one_stream_call(update):
    """forward_segment per segment, a small internal window, and one forward_stream call
    give the same result (to rounding: the chunking of the state pass may differ)."""
    gu.require_gpu()
    w = wl.Workload(f"split-{update}", 1, 3, 128, 256, 5 * 256, "bf16", update, seed=9)
    gu.note(f"[parity] call split {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    ref = _run_case(w, beta, Q, K, V, want_parts=False)
    win = _run_case(w, beta, Q, K, V, want_parts=False, max_window_segments=2)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    with binding.InfiniAttention(1, 3, 128, 256, update=update, beta=beta) as layer:
        outs = [layer.forward_segment(*(x[:, :, s:s + 256].contiguous() for x in dev))
                for s in range(0, 5 * 256, 256)]
        M, z = layer.get_state()
        seg = dict(out=torch.cat(outs, dim=2).float().cpu().numpy(), M=M.cpu().numpy(), z=z.cpu().numpy())
    for other in (win, seg):
        d_out = np.abs(other["out"] - ref["out"]).max()
        assert d_out <= 2 * 2**-8 * np.abs(ref["out"]).max(), d_out
        assert gu.rel(other["M"], ref["M"]) <= 1e-5
        assert gu.rel(other["z"], ref["z"]) <= 1e-6


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_state_save_restore_is_bit_identical(update):
    gu.require_gpu()
    w = wl.Workload(f"resume-{update}", 2, 2, 128, 256, 6 * 256, "bf16", update, seed=10)
    gu.note(f"[parity] resume {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    first = [x[:, :, :512].contiguous() for x in dev]
    second = [x[:, :, 512:].contiguous() for x in dev]
    with binding.InfiniAttention(2, 2, 128, 256, update=update, beta=beta) as a:
        a.forward_stream(*first)
        out_a = a.forward_stream(*second)
        Ma, za = a.get_state()
    with binding.InfiniAttention(2, 2, 128, 256, update=update, beta=beta) as b:
        b.forward_stream(*first)
        Ms, zs = b.get_state()
        b.reset_state()
        Mr, zr = b.get_state()
        assert torch.count_nonzero(Mr) == 0 and torch.count_nonzero(zr) == 0
        b.set_state(Ms, zs)
        out_b = b.forward_stream(*second)
        Mb, zb = b.get_state()
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(Ma, Mb) and torch.equal(za, zb)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_reset_between_streams(update):
    """reset_state enqueues nothing: the next forward must read the state as zero (it
    equals a fresh handle), and a partial set_state after a reset keeps the other part 0."""
    gu.require_gpu()
    w = wl.Workload(f"reset-{update}", 1, 2, 128, 256, 3 * 256 + 40, "bf16", update, seed=13)
    gu.note(f"[parity] reset between streams {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    with binding.InfiniAttention(1, 2, 128, 256, update=update, beta=beta) as fresh:
        out_f = fresh.forward_stream(*dev)
        Mf, zf = fresh.get_state()
    with binding.InfiniAttention(1, 2, 128, 256, update=update, beta=beta) as layer:
        layer.forward_stream(*dev)
        layer.forward_stream(*dev)
        layer.reset_state()
        out_r = layer.forward_stream(*dev)
        Mr, zr = layer.get_state()
        layer.reset_state()
        layer.set_state(torch.ones_like(Mr), None)
        M1, z1 = layer.get_state()
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_r)
    assert torch.equal(Mf, Mr) and torch.equal(zf, zr)
    assert torch.all(M1 == 1) and torch.count_nonzero(z1) == 0


def test_nonzero_initial_state_and_literal_scale():
    """set_state with an arbitrary start, and the page's literal 1/sqrt(d_model) scale."""
    gu.require_gpu()
    B, H, d, N, L = 1, 2, 128, 256, 600
    w = wl.Workload("init-state", B, H, d, N, L, "bf16", "delta", seed=12)
    gu.note("[parity] nonzero initial state, scale 1/sqrt(H*d)")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    rng = np.random.default_rng(3)
    z0 = (np.abs(rng.standard_normal((B, H, d))) * 50 + 100).astype(np.float32)
    M0 = (rng.standard_normal((B, H, d, d)) * 5).astype(np.float32)
    scale = float(1.0 / np.sqrt(H * d))
    with binding.InfiniAttention(B, H, d, N, update="delta", beta=beta, softmax_scale=scale) as layer:
        layer.set_state(torch.from_numpy(M0), torch.from_numpy(z0))
        out = layer.forward_stream(*[gu.to_dev(x, "bf16") for x in (Q, K, V)])
        M, z = layer.get_state()
    O_ref, M_ref, z_ref = orc.forward(Q, K, V, beta, N, "delta", eps=w.eps, scale=scale, M0=M0, z0=z0)
    gu.check_output(out.float().cpu().numpy(), O_ref, gu.BF16_TOL)
    gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, gu.BF16_TOL)


@pytest.mark.parametrize("B,H,d,N,L,io,update", [
    (1, 3, 128, 256, 3 * 256 + 77, "bf16", "linear"),
    (2, 2, 128, 512, 2 * 512 + 300, "bf16", "delta"),
    (1, 2, 64, 192, 2 * 192 + 1, "bf16", "linear"),
    (1, 2, 128, 96, 3 * 96 + 5, "f32", "delta"),
])
def test_separate_local_qk_matches_oracle(B, H, d, N, L, io, update):
    """Position-embedded Q/K for the local attention only (RoPE applied by the caller),
    PE-free Q/K for the memory: forward_stream_local against the oracle."""
    gu.require_gpu()
    w = wl.Workload(f"local-qk-{io}-{update}-d{d}", B, H, d, N, L, io, update, seed=14)
    gu.note(f"[parity] local Q/K {w.name}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    Ql, Kl = rope(Q), rope(K)
    if io == "bf16":
        Ql, Kl = wl.round_to_bf16(Ql), wl.round_to_bf16(Kl)
    else:
        Ql, Kl = Ql.astype(np.float32), Kl.astype(np.float32)
    dev = [gu.to_dev(x, io) for x in (Q, K, V, Ql, Kl)]
    with binding.InfiniAttention(B, H, d, N, update=update, io_dtype=io, eps=w.eps, beta=beta) as layer:
        out = layer.forward_stream_local(*dev)
        M, z = layer.get_state()
    O_ref, M_ref, z_ref = orc.forward(Q, K, V, beta, N, update, eps=w.eps, Q_local=Ql, K_local=Kl)
    tol = gu.tol_for(io)
    gu.check_output(out.float().cpu().numpy(), O_ref, tol)
    gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, tol)
