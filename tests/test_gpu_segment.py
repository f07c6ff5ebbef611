"""GPU parity of one-segment calls (the streaming path: one forward_segment per segment)
through the C-ABI against the CPU oracle.

With few (batch, head) pairs a one-segment call splits the keys of each 256-query tile into
chunks handled by different workgroups (the last one to finish merges the partial softmax
states in chunk order), reads the carried state from its bf16 M^T copy, and runs the
memory-update kernels on a second stream (the chain, which writes the new state, is joined
by the next call that needs it).  These tests cover that path at the workload shape (8
heads, d = 128, N = 2048: query tiles split into up to four chunks), at d = 64, on ragged
segments, after reset_state and set_state, mixed with the other calls on one handle, and
its run-to-run determinism.
Tolerances are in tests/gpu_util.py."""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from oracle import infini_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _per_segment(w, beta, Q, K, V, seg_lens, M0=None, z0=None, reset_first=False):
    """Feed the stream one forward_segment call per entry of seg_lens; returns the
    concatenated output and the final state."""
    dev = [gu.to_dev(x, w.io_dtype) for x in (Q, K, V)]
    with binding.InfiniAttention(w.batch, w.heads, w.head_dim, w.segment_len, update=w.update,
                                 io_dtype=w.io_dtype, eps=w.eps, beta=beta) as layer:
        if reset_first:   # a first stream, then a reset: the next call must read a zero state
            layer.forward_segment(*(x[:, :, :seg_lens[0]].contiguous() for x in dev))
            layer.reset_state()
        if M0 is not None:
            layer.set_state(torch.from_numpy(M0).cuda(), torch.from_numpy(z0).cuda())
        outs, lo = [], 0
        for n in seg_lens:
            outs.append(layer.forward_segment(*(x[:, :, lo:lo + n].contiguous() for x in dev)))
            lo += n
        M, z = layer.get_state()
        torch.cuda.synchronize()
        return (torch.cat(outs, dim=2).float().cpu().numpy(), M.cpu().numpy(), z.cpu().numpy())


CASES = [
    # name, B, H, d, N, segment lengths, update
    ("h8-d128-n2048-linear", 1, 8, 128, 2048, (2048, 2048, 1000), "linear"),
    ("h8-d128-n2048-delta", 1, 8, 128, 2048, (2048, 2048, 1000), "delta"),
    ("b2-h2-d64-n1024-linear", 2, 2, 64, 1024, (1024, 700, 1024), "linear"),
    ("b2-h2-d64-n1024-delta", 2, 2, 64, 1024, (1024, 1024, 333), "delta"),
    ("h3-d128-n2048-ragged", 1, 3, 128, 2048, (1, 65, 300, 2047, 2048), "linear"),
    # 4K segments: split-key calls with 8 key chunks on the last query tiles
    ("h2-d128-n4096-linear", 1, 2, 128, 4096, (4096, 2500), "linear"),
    ("h2-d128-n4096-delta", 1, 2, 128, 4096, (4096, 4096, 1500), "delta"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_segment_calls_match_oracle(case):
    gu.require_gpu()
    name, B, H, d, N, lens, update = case
    L = sum(lens)
    w = wl.Workload(name, B, H, d, N, L, "bf16", update, seed=71)
    gu.note(f"[segment] {name}: B={B} H={H} d={d} N={N} segments {lens} {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    out, M, z = _per_segment(w, beta, Q, K, V, lens)
    # the oracle segment by segment (calls of fewer than N tokens are segments of their own)
    M_ref = np.zeros((B, H, d, d))
    z_ref = np.zeros((B, H, d))
    lo = 0
    for s, n in enumerate(lens):
        o_ref, M_ref, z_ref = orc.forward(Q[:, :, lo:lo + n], K[:, :, lo:lo + n], V[:, :, lo:lo + n], beta, N,
                                          update, eps=w.eps, M0=M_ref, z0=z_ref)
        gu.check_output(out[:, :, lo:lo + n], o_ref, gu.BF16_TOL, f"out segment {s}")
        lo += n
    gu.check_state(M, z, M_ref, z_ref, gu.BF16_TOL)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_segment_calls_after_reset_and_set_state(update):
    """reset_state before a one-segment call: the call reads a zero state (its bf16 copy
    of M^T is not consulted); set_state: the copy is rebuilt from the new M."""
    gu.require_gpu()
    B, H, d, N = 1, 4, 128, 2048
    lens = (2048, 1500)
    w = wl.Workload(f"seg-reset-{update}", B, H, d, N, sum(lens), "bf16", update, seed=72)
    gu.note(f"[segment] reset / set_state {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    fresh = _per_segment(w, beta, Q, K, V, lens)
    after_reset = _per_segment(w, beta, Q, K, V, lens, reset_first=True)
    for a, b in zip(fresh, after_reset):
        assert np.array_equal(a, b)
    # a state as an earlier stream would leave it
    _, M0, z0 = orc.forward(*wl.stream_inputs(wl.Workload("seg-pre", B, H, d, N, 2 * N, "bf16", update, seed=73)),
                            beta, N, update, eps=w.eps)
    M0, z0 = M0.astype(np.float32), z0.astype(np.float32)
    out, M, z = _per_segment(w, beta, Q, K, V, lens, M0=M0, z0=z0)
    M_ref, z_ref, lo = M0.astype(np.float64), z0.astype(np.float64), 0
    for s, n in enumerate(lens):
        o_ref, M_ref, z_ref = orc.forward(Q[:, :, lo:lo + n], K[:, :, lo:lo + n], V[:, :, lo:lo + n], beta, N,
                                          update, eps=w.eps, M0=M_ref, z0=z_ref)
        gu.check_output(out[:, :, lo:lo + n], o_ref, gu.BF16_TOL, f"out segment {s} after set_state")
        lo += n
    gu.check_state(M, z, M_ref, z_ref, gu.BF16_TOL)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_segment_calls_are_deterministic_and_agree_with_forward_stream(update):
    """Three runs of the split-key path give identical bits; one forward_stream call over
    the same stream agrees to rounding (the chunked softmax adds in another order)."""
    gu.require_gpu()
    B, H, d, N = 1, 8, 128, 2048
    lens = (2048, 2048, 2048)
    w = wl.Workload(f"seg-det-{update}", B, H, d, N, sum(lens), "bf16", update, seed=74)
    gu.note(f"[segment] determinism {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    runs = [_per_segment(w, beta, Q, K, V, lens) for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert np.array_equal(a, b)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    with binding.InfiniAttention(B, H, d, N, update=update, eps=w.eps, beta=beta) as layer:
        ref = layer.forward_stream(*dev).float().cpu().numpy()
        M, z = layer.get_state()
        M, z = M.cpu().numpy(), z.cpu().numpy()
    out = runs[0][0]
    d_out = float(np.abs(out - ref).max())
    assert d_out <= 2 * 2**-8 * float(np.abs(ref).max()), d_out
    assert gu.rel(runs[0][1], M) <= 1e-5
    assert gu.rel(runs[0][2], z) <= 1e-6


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_mixed_calls_on_one_handle(update):
    """One handle, one stream: forward_segment, a two-segment forward_stream, forward_segment
    again, then token-by-token decoding and a flush.  Each call must see the state the
    previous one left (the one-segment calls leave their memory update running on the
    second stream), and the whole equals the oracle over the same segmentation."""
    gu.require_gpu()
    B, H, d, N = 1, 8, 128, 2048
    n_dec = 5
    L = 4 * N + n_dec
    w = wl.Workload(f"seg-mixed-{update}", B, H, d, N, L, "bf16", update, seed=75)
    gu.note(f"[segment] mixed calls {update}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    sl = lambda lo, hi: [x[:, :, lo:hi].contiguous() for x in dev]   # noqa: E731
    with binding.InfiniAttention(B, H, d, N, update=update, eps=w.eps, beta=beta) as layer:
        outs = [layer.forward_segment(*sl(0, N)), layer.forward_stream(*sl(N, 3 * N)),
                layer.forward_segment(*sl(3 * N, 4 * N))]
        for t in range(4 * N, L):
            outs.append(layer.decode_step(*(x[:, :, t].contiguous() for x in dev))[:, :, None])
        layer.decode_flush()
        M, z = layer.get_state()
        torch.cuda.synchronize()
        out = torch.cat(outs, dim=2).float().cpu().numpy()
        M, z = M.cpu().numpy(), z.cpu().numpy()
    o_ref, M_ref, z_ref = orc.forward(Q, K, V, beta, N, update, eps=w.eps)
    gu.check_output(out, o_ref, gu.BF16_TOL, "out")
    gu.check_state(M, z, M_ref, z_ref, gu.BF16_TOL)
