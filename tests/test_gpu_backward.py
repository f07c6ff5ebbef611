"""GPU parity of the backward pass (gradients back through the M / z recurrence) through
the C-ABI against the CPU backward oracle (float64 autograd of the layer), plus
full-size properties.

Tolerances, against the oracle, for every gradient tensor:
* relative Frobenius error <= 2e-2 with bf16 inputs (the recomputed forward rounds P and
  M_{s-1} to bf16 as the forward does, the gradient products take bf16 operands and the
  upstream gradient is bf16), <= 1e-4 on the all-float32 path; over the whole tensor and
  separately for every (batch, head) and, for the per-token gradients, every (batch, head,
  segment) block;
* element by element: max |got - ref| within the same fraction (2e-2, 1e-4) of the
  largest |ref| of its block, so that one wrong tile or segment cannot hide in a norm.
  (bf16 operand rounding is 2^-9 relative per element and averages out over a
  contraction, so the elements stay within a few 1e-3 of the block maximum.)
"""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from oracle import infini_backward as ob
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GRAD_TOL = {"bf16": 2e-2, "f32": 1e-4}


def _check_block(got, ref, tol, what, whole=None):
    """Relative Frobenius error and max-abs error against the block's maximum.  A block
    whose exact gradient is far below the tensor's scale -- a one-token segment, where the
    retrieval's numerator and denominator terms cancel almost exactly -- is measured
    against 10% of an average block of the whole tensor instead (``whole``: the full
    reference): rounding of the cancelling terms is relative to their size, not to the
    tiny difference."""
    nb = float(np.linalg.norm(ref))
    scale = float(np.abs(ref).max())
    if whole is not None:
        nb = max(nb, 0.1 * float(np.linalg.norm(whole)) * np.sqrt(ref.size / whole.size))
        scale = max(scale, 0.1 * float(np.abs(whole).max()))
    dn = float(np.linalg.norm(got - ref))
    r = dn / nb if nb > 0 else dn
    assert r <= tol, f"{what}: relative error {r:.3e} > {tol}"
    err = float(np.abs(got - ref).max())
    assert err <= tol * scale or (scale == 0.0 and err == 0.0), \
        f"{what}: max-abs {err:.3e} > {tol} x block max {scale:.3e}"
    return r, (err / scale if scale > 0 else 0.0)


def _check_grad(got, ref, tol, what, seg_len=None):
    """Whole tensor, then every (batch, head) block (leading two axes of a [B, H, ...]
    tensor), then for [B, H, L, d] tensors with seg_len given every (batch, head, segment)
    block: relative Frobenius error and element-wise max-abs against the block maximum."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = list(_check_block(got, ref, tol, what))
    if got.ndim >= 3:
        for b in range(got.shape[0]):
            for h in range(got.shape[1]):
                blocks = [(f"b{b} h{h}", slice(None))]
                if seg_len is not None and got.ndim == 4:
                    L = got.shape[2]
                    blocks = [(f"b{b} h{h} tokens {lo}:{min(lo + seg_len, L)}", slice(lo, min(lo + seg_len, L)))
                              for lo in range(0, L, seg_len)]
                for name, sl in blocks:
                    r, e = _check_block(got[b, h, sl], ref[b, h, sl], tol, f"{what} {name}", whole=ref)
                    worst = [max(worst[0], r), max(worst[1], e)]
    return worst


CASES = [
    # name, B, H, d, N, L, dtype, update, with initial state, with final-state gradient
    ("bf16-linear-d128", 1, 2, 128, 128, 3 * 128 + 29, "bf16", "linear", False, False),
    ("bf16-delta-d128", 1, 2, 128, 128, 3 * 128 + 29, "bf16", "delta", False, False),
    ("bf16-linear-d64-state", 2, 2, 64, 96, 2 * 96 + 40, "bf16", "linear", True, True),
    ("bf16-delta-d64-state", 2, 1, 64, 96, 2 * 96 + 40, "bf16", "delta", True, True),
    # several 128-key tiles per segment and a ragged last tile (the linear rule's fused epilogue)
    ("bf16-linear-d128-n320-state", 1, 2, 128, 320, 2 * 320 + 77, "bf16", "linear", True, True),
    # two and three 512-token chunks of the R pass per segment (the chains' register paths)
    ("bf16-linear-d64-n1024-state", 1, 1, 64, 1024, 2 * 1024 + 100, "bf16", "linear", True, True),
    ("bf16-linear-d64-n1100", 1, 1, 64, 1100, 2 * 1100 + 9, "bf16", "linear", False, True),
    ("f32-linear-d128", 1, 2, 128, 64, 2 * 64 + 17, "f32", "linear", True, True),
    ("f32-delta-d128", 1, 2, 128, 64, 2 * 64 + 17, "f32", "delta", True, True),
    ("f32-delta-d64-n1", 1, 2, 64, 1, 5, "f32", "delta", False, True),
    # the shapes the throughput workloads run: d=128, N=2048 (four 512-token chunks of the R
    # pass, the delta rule's 128-token update tiles), four full segments and a ragged fifth,
    # the gate open, an initial state and gradients of the final state
    ("bf16-linear-d128-n2048-bench", 1, 2, 128, 2048, 4 * 2048 + 300, "bf16", "linear", True, True),
    ("bf16-delta-d128-n2048-bench", 1, 2, 128, 2048, 4 * 2048 + 300, "bf16", "delta", True, True),
    # calls longer than one internal window (the last field: segments per window): the state
    # at every window start recorded forward, the windows run in reverse
    ("bf16-linear-d128-win2", 1, 2, 128, 256, 5 * 256 + 40, "bf16", "linear", True, True, 2),
    ("bf16-delta-d128-win2", 2, 1, 128, 256, 5 * 256 + 40, "bf16", "delta", False, True, 2),
    ("f32-delta-d64-win1", 1, 2, 64, 64, 3 * 64 + 5, "f32", "delta", True, True, 1),
    ("bf16-linear-d128-n2048-win2", 1, 2, 128, 2048, 4 * 2048 + 300, "bf16", "linear", True, True, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    gu.require_gpu()
    name, B, H, d, N, L, dtype, update, with_state, with_dstate = case[:10]
    win = case[10] if len(case) > 10 else 0
    gu.note(f"[backward] {name}: B={B} H={H} d={d} N={N} L={L} {dtype} {update} window {win or 'default'}")
    w = wl.Workload(name, B, H, d, N, L, dtype, update, seed=61)
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    rng = np.random.default_rng(62)
    dO = rng.standard_normal((B, H, L, d)).astype(np.float32)
    if dtype == "bf16":
        dO = wl.round_to_bf16(dO)
    M0 = z0 = dM = dz = None
    if with_state:   # a state as a previous stream would leave it
        _, M0, z0 = ob.forward_torch(*(torch.tensor(x, dtype=torch.float64) for x in wl.stream_inputs(
            wl.Workload(name + "-pre", B, H, d, N, 2 * N, dtype, update, seed=63))),
            torch.tensor(beta, dtype=torch.float64), N, update)
        M0, z0 = M0.numpy().astype(np.float32), z0.numpy().astype(np.float32)
    if with_dstate:
        dM = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
        dz = (rng.standard_normal((B, H, d)) * 0.05).astype(np.float32)
    dev = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda")   # noqa: E731
    with binding.InfiniAttention(B, H, d, N, update=update, io_dtype=dtype, eps=w.eps, beta=beta,
                                 max_window_segments=win) as layer:
        res = layer.backward(*(gu.to_dev(x, dtype) for x in (Q, K, V, dO)), m0=dev(M0), z0=dev(z0),
                             dm_final=dev(dM), dz_final=dev(dz))
        torch.cuda.synchronize()
        got = {k_: t.cpu().numpy() for k_, t in res.items()}
    ref = ob.gradients(Q, K, V, beta, dO, N, update, w.eps, None, M0, z0, dM, dz)
    tol = GRAD_TOL[dtype]
    for gname, rname in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV"), ("dbeta", "dbeta"), ("dm0", "dM0"),
                         ("dz0", "dz0")):
        r, e = _check_grad(got[gname], ref[rname], tol, gname, seg_len=N if gname in ("dq", "dk", "dv") else None)
        gu.note(f"  {gname}: worst block rel {r:.2e}, worst max-abs / block max {e:.2e}")


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_backward_is_deterministic(update):
    """Batch 4, 2 heads, d=128, N=2048, three segments (the last ragged): three backward
    calls on the same inputs give bit-identical gradients (every partial sum is taken in a
    fixed order; no float atomics)."""
    gu.require_gpu()
    B, H, d, N, L = 4, 2, 128, 2048, 2 * 2048 + 700
    gu.note(f"[backward] determinism {update}: B={B} H={H} d={d} N={N} L={L}")
    w = wl.Workload(f"bwd-det-{update}", B, H, d, N, L, "bf16", update, seed=67)
    dev = [gu.to_dev(x, "bf16") for x in wl.stream_inputs(w)]
    rng = np.random.default_rng(68)
    d_out = gu.to_dev(rng.standard_normal((B, H, L, d)).astype(np.float32), "bf16")
    dmf = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)).to("cuda")
    dzf = torch.from_numpy((rng.standard_normal((B, H, d)) * 0.05).astype(np.float32)).to("cuda")
    with binding.InfiniAttention(B, H, d, N, update=update, eps=w.eps, beta=wl.beta_for(w)) as layer:
        runs = []
        for _ in range(3):
            g = layer.backward(*dev, d_out, dm_final=dmf, dz_final=dzf)
            torch.cuda.synchronize()
            runs.append({k_: t.cpu().clone() for k_, t in g.items()})
    for k_ in runs[0]:
        for r in runs[1:]:
            assert torch.equal(runs[0][k_].view(torch.int32), r[k_].view(torch.int32)), f"{k_} differs between runs"


def test_backward_leaves_the_handle_state_alone():
    gu.require_gpu()
    B, H, d, N, L = 1, 2, 64, 64, 150
    w = wl.Workload("bwd-state", B, H, d, N, L, "bf16", "linear", seed=64)
    Q, K, V = (gu.to_dev(x, "bf16") for x in wl.stream_inputs(w))
    with binding.InfiniAttention(B, H, d, N, eps=w.eps, beta=wl.beta_for(w)) as layer:
        layer.forward_stream(Q, K, V)
        M1, z1 = layer.get_state()
        layer.backward(Q, K, V, torch.ones_like(Q))
        M2, z2 = layer.get_state()
        torch.cuda.synchronize()
        assert torch.equal(M1, M2) and torch.equal(z1, z2)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_full_size_backward_properties(update):
    """8 heads, d=128, N=2048, 32K tokens: (1) with the gate closed (beta = -inf) and no
    state gradient, sampled heads and segments of dQ, dK, dV equal causal attention's
    gradient (float32 on the CPU); (2) the gradients are linear in the upstream gradient."""
    gu.require_gpu()
    base = wl.WORKLOADS[wl.THROUGHPUT_WORKLOAD]
    w = wl.Workload(base.name + "-" + update, 1, base.heads, base.head_dim, base.segment_len, base.n_tokens,
                    "bf16", update, seed=base.seed)
    H, d, N, L = w.heads, w.head_dim, w.segment_len, w.n_tokens
    gu.note(f"[backward] full size {w.name}")
    Q, K, V = wl.stream_inputs(w)
    rng = np.random.default_rng(65)
    dO1 = wl.round_to_bf16(rng.standard_normal((1, H, L, d)).astype(np.float32))
    dO2 = wl.round_to_bf16(rng.standard_normal((1, H, L, d)).astype(np.float32))
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    with binding.InfiniAttention(1, H, d, N, update=update, eps=w.eps, beta=[-np.inf] * H) as closed:
        g = closed.backward(*dev, gu.to_dev(dO1, "bf16"))
        torch.cuda.synchronize()
        for h, s in ((0, 0), (3, 7), (7, L // N - 1)):
            lo, hi = s * N, (s + 1) * N
            q, k, v = (torch.tensor(x[0, h, lo:hi], dtype=torch.float32, requires_grad=True) for x in (Q, K, V))
            o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
            dq, dk, dv = torch.autograd.grad((o * torch.tensor(dO1[0, h, lo:hi])).sum(), [q, k, v])
            for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
                _check_grad(g[name][0, h, lo:hi].cpu().numpy(), ref.numpy(), 2e-2, f"{name} h{h} s{s}")
    beta = wl.beta_for(w)
    with binding.InfiniAttention(1, H, d, N, update=update, eps=w.eps, beta=beta) as layer:
        ga = layer.backward(*dev, gu.to_dev(dO1, "bf16"))
        gb = layer.backward(*dev, gu.to_dev(dO2, "bf16"))
        gs = layer.backward(*dev, gu.to_dev(dO1 + dO2, "bf16"))   # sums of two bf16 values: rounded once more
        torch.cuda.synchronize()
        for name in ("dq", "dk", "dv", "dbeta", "dm0", "dz0"):
            _check_grad((gs[name]).cpu().numpy(), (ga[name] + gb[name]).cpu().numpy(), 2e-2, f"linearity {name}")


def test_full_size_linear_update_gradients_closed_form():
    """8 heads, d=128, N=2048, 32K tokens, linear rule, gate closed (beta = -inf) and dO = 0:
    only <dm_final, M_final> + <dz_final, z_final> carry gradient.  The retrieval then passes
    none back (g = 0), so dL/dM_s = dm_final and dL/dz_s = dz_final for every segment (Eq. 8
    differentiated: M_s = M_{s-1} + sigma(K_s)^T V_s, z_s = z_{s-1} + sum_t sigma(k_t)), and per
    token dV_t = sigma(k_t) dm_final and dK_t = (dm_final v_t + dz_final) o sigma'(k_t) — the
    part the dK, dV kernel adds in its epilogue, checked here on sampled tokens of every
    segment against float64 on the CPU."""
    gu.require_gpu()
    base = wl.WORKLOADS[wl.THROUGHPUT_WORKLOAD]
    w = wl.Workload(base.name + "-linear", 1, base.heads, base.head_dim, base.segment_len, base.n_tokens,
                    "bf16", "linear", seed=base.seed)
    H, d, N, L = w.heads, w.head_dim, w.segment_len, w.n_tokens
    gu.note(f"[backward] closed-form update gradients {w.name}")
    Q, K, V = wl.stream_inputs(w)
    rng = np.random.default_rng(66)
    dmf = rng.standard_normal((1, H, d, d)).astype(np.float32)
    dzf = rng.standard_normal((1, H, d)).astype(np.float32)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    d_out = gu.to_dev(np.zeros((1, H, L, d), dtype=np.float32), "bf16")
    with binding.InfiniAttention(1, H, d, N, update="linear", eps=w.eps, beta=[-np.inf] * H) as layer:
        g = layer.backward(*dev, d_out, dm_final=torch.from_numpy(dmf), dz_final=torch.from_numpy(dzf))
        torch.cuda.synchronize()
    dk, dv, dq = (g[n].cpu().numpy() for n in ("dk", "dv", "dq"))
    assert np.all(dq == 0.0), "dQ must vanish with dO = 0 and the gate closed"
    toks = np.concatenate([s * N + np.array([0, 1, 63, 64, 127, 128, 1000, N - 1]) for s in range(L // N)])
    for h in (0, 5, H - 1):
        k64 = K[0, h, toks].astype(np.float64)
        v64 = V[0, h, toks].astype(np.float64)
        sig = np.where(k64 > 0, k64 + 1.0, np.exp(k64))
        dsig = np.where(k64 > 0, 1.0, np.exp(k64))
        m = dmf[0, h].astype(np.float64)
        ref_dv = sig @ m
        ref_dk = (v64 @ m.T + dzf[0, h].astype(np.float64)) * dsig
        _check_grad(dv[0, h, toks], ref_dv, 2e-2, f"dv h{h}")
        _check_grad(dk[0, h, toks], ref_dk, 2e-2, f"dk h{h}")


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_full_size_multi_window_backward_agrees_with_one_window(update):
    """2 heads, d=128, N=2048, 32 segments (64K tokens): the backward of the whole stream
    as one internal window and as four windows of 8 segments (states recorded at the
    window starts, windows run in reverse, the state gradient handed back between them)
    agree to rounding, with an initial state and final-state gradients."""
    gu.require_gpu()
    B, H, d, N, S = 1, 2, 128, 2048, 32
    w = wl.Workload(f"bwd-multiwin-{update}", B, H, d, N, S * N, "bf16", update, seed=69)
    gu.note(f"[backward] full size, 4 windows vs 1: {update}")
    dev = [gu.to_dev(x, "bf16") for x in wl.stream_inputs(w)]
    rng = np.random.default_rng(70)
    d_out = gu.to_dev(rng.standard_normal((B, H, S * N, d)).astype(np.float32), "bf16")
    m0 = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.02).astype(np.float32)).cuda()
    z0 = torch.from_numpy(np.abs(rng.standard_normal((B, H, d)) * 100).astype(np.float32)).cuda()
    dmf = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)).cuda()
    dzf = torch.from_numpy((rng.standard_normal((B, H, d)) * 0.05).astype(np.float32)).cuda()
    res = {}
    for win in (32, 8):
        with binding.InfiniAttention(B, H, d, N, update=update, eps=w.eps, beta=wl.beta_for(w),
                                     max_window_segments=win) as layer:
            g = layer.backward(*dev, d_out, m0=m0, z0=z0, dm_final=dmf, dz_final=dzf)
            torch.cuda.synchronize()
            res[win] = {k_: t.cpu().numpy() for k_, t in g.items()}
            del g
    for k_ in res[32]:
        _check_grad(res[8][k_], res[32][k_], 1e-3, f"{k_} (4 windows vs 1)",
                    seg_len=N if k_ in ("dq", "dk", "dv") else None)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_backward_scratch_reuse_with_a_short_last_segment(update):
    """One handle, two backward calls: a long one (every token tile of every segment
    written), then one whose last segment is short.  The second reuses the scratch of the
    first; per-tile partials of the tiles past the short segment's end must not leak in.
    Both start from a carried state, as in training.  (From a zero state the delta rule's
    first-segment dV is a small residual -- the second segment's update nearly erases the
    first one's contribution -- and its per-segment error against float64 reaches ~2.5%.)"""
    gu.require_gpu()
    B, H, d, N = 1, 2, 128, 2048
    beta = wl.beta_for(wl.Workload("reuse", B, H, d, N, N, "bf16", update, seed=76))
    _, M0, z0 = ob.forward_torch(*(torch.tensor(x, dtype=torch.float64) for x in wl.stream_inputs(
        wl.Workload("reuse-pre", B, H, d, N, 2 * N, "bf16", update, seed=63))),
        torch.tensor(beta, dtype=torch.float64), N, update)
    M0, z0 = M0.numpy().astype(np.float32), z0.numpy().astype(np.float32)
    with binding.InfiniAttention(B, H, d, N, update=update, eps=1e-6, beta=beta) as layer:
        for L, seed in ((2 * N, 77), (N + 40, 78)):
            w = wl.Workload(f"reuse-{update}-{L}", B, H, d, N, L, "bf16", update, seed=seed)
            gu.note(f"[backward] scratch reuse {update}: L={L}")
            Q, K, V = wl.stream_inputs(w)
            rng = np.random.default_rng(seed)
            dO = wl.round_to_bf16(rng.standard_normal((B, H, L, d)).astype(np.float32))
            dM = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
            dz = (rng.standard_normal((B, H, d)) * 0.05).astype(np.float32)
            res = layer.backward(*(gu.to_dev(x, "bf16") for x in (Q, K, V, dO)),
                                 m0=torch.from_numpy(M0).cuda(), z0=torch.from_numpy(z0).cuda(),
                                 dm_final=torch.from_numpy(dM).cuda(), dz_final=torch.from_numpy(dz).cuda())
            torch.cuda.synchronize()
            got = {k_: t.cpu().numpy() for k_, t in res.items()}
            ref = ob.gradients(Q, K, V, beta, dO, N, update, w.eps, None, M0, z0, dM, dz)
            for gname, rname in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV"), ("dbeta", "dbeta"), ("dm0", "dM0"),
                                 ("dz0", "dz0")):
                _check_grad(got[gname], ref[rname], GRAD_TOL["bf16"], f"{gname} L={L}",
                            seg_len=N if gname in ("dq", "dk", "dv") else None)
