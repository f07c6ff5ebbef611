"""GPU parity of incremental decoding (one token per sequence per call) through the C-ABI
against the oracle's token-by-token definition, plus the rules around an open segment.
Tolerances are those of the per-head tests (tests/gpu_util.py)."""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from oracle import infini_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _decode_all(layer, Q, K, V, io_dtype, flush=True):
    """Feeds [B, H, L, d] inputs token by token; returns the outputs [B, H, L, d]."""
    dev = [gu.to_dev(x, io_dtype) for x in (Q, K, V)]
    L = Q.shape[2]
    outs = []
    for t in range(L):
        q, k, v = (x[:, :, t].contiguous() for x in dev)
        outs.append(layer.decode_step(q, k, v))
    if flush:
        layer.decode_flush()
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2).float().cpu().numpy()


CASES = [
    # name, B, H, d, N, L, dtype, update
    ("bf16-linear-d128", 2, 2, 128, 64, 2 * 64 + 37, "bf16", "linear"),
    ("bf16-delta-d128", 2, 2, 128, 64, 2 * 64 + 37, "bf16", "delta"),
    ("bf16-linear-d64-n48", 1, 3, 64, 48, 3 * 48 + 5, "bf16", "linear"),
    ("bf16-delta-d64-n1", 1, 2, 64, 1, 6, "bf16", "delta"),
    ("bf16-linear-n300", 1, 2, 128, 300, 310, "bf16", "linear"),   # several key rounds per token
    ("f32-linear-d128", 1, 2, 128, 40, 2 * 40 + 9, "f32", "linear"),
    ("f32-delta-d64", 2, 1, 64, 32, 3 * 32, "f32", "delta"),
    # few (batch, head) pairs and more than 128 cached keys: the keys split over workgroups
    ("bf16-delta-d64-n260-split", 1, 2, 64, 260, 270, "bf16", "delta"),
    ("f32-linear-n300-split", 1, 2, 128, 300, 310, "f32", "linear"),
    # 4K segments: up to 16 chunks of 256 keys per pair, the most a token splits into
    ("bf16-linear-n4096-split16", 1, 1, 128, 4096, 4096 + 300, "bf16", "linear"),
    ("bf16-delta-n4096-split16", 1, 1, 128, 4096, 4096 + 40, "bf16", "delta"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(case):
    gu.require_gpu()
    name, B, H, d, N, L, dtype, update = case
    gu.note(f"[decode] {name}: B={B} H={H} d={d} N={N} L={L} {dtype} {update}")
    w = wl.Workload(name, B, H, d, N, L, dtype, update, seed=51)
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    with binding.InfiniAttention(B, H, d, N, update=update, io_dtype=dtype, eps=w.eps, beta=beta) as layer:
        out = _decode_all(layer, Q, K, V, dtype)
        assert layer.decode_position() == 0
        M, z = layer.get_state()
        torch.cuda.synchronize()
    O_ref, M_ref, z_ref, open_tokens = orc.decode_stream(Q, K, V, beta, N, update, eps=w.eps)
    assert open_tokens == 0
    tol = gu.tol_for(dtype)
    gu.check_output(out, O_ref, tol)
    gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, tol)


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_decode_agrees_with_forward_stream(update):
    """The same stream through forward_stream and token by token: outputs within the bf16
    tolerance of each other, states within the fp32 state tolerance."""
    gu.require_gpu()
    B, H, d, N, L = 2, 2, 128, 128, 3 * 128
    gu.note(f"[decode] vs forward_stream, {update}")
    w = wl.Workload("dec-vs-stream", B, H, d, N, L, "bf16", update, seed=52)
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    kw = dict(update=update, eps=w.eps, beta=beta)
    with binding.InfiniAttention(B, H, d, N, **kw) as dec, binding.InfiniAttention(B, H, d, N, **kw) as stm:
        out_d = _decode_all(dec, Q, K, V, "bf16")
        out_s = stm.forward_stream(*(gu.to_dev(x, "bf16") for x in (Q, K, V))).float().cpu().numpy()
        Md, zd = dec.get_state()
        Ms, zs = stm.get_state()
        torch.cuda.synchronize()
    tol = gu.tol_for("bf16")
    gu.check_output(out_d, out_s, tol, "decode vs stream")
    gu.check_state(Md.cpu().numpy(), zd.cpu().numpy(), Ms.cpu().numpy(), zs.cpu().numpy(), tol)


def test_open_segment_rules():
    gu.require_gpu()
    B, H, d, N = 1, 2, 64, 16
    w = wl.Workload("dec-rules", B, H, d, N, 2 * N + 5, "bf16", "linear", seed=53)
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    with binding.InfiniAttention(B, H, d, N, eps=w.eps, beta=beta) as layer:
        dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
        tok = lambda t: [x[:, :, t].contiguous() for x in dev]   # noqa: E731
        for t in range(N + 3):
            layer.decode_step(*tok(t))
        assert layer.decode_position() == 3
        with pytest.raises(binding.InfiniAttnError):
            layer.forward_stream(*dev)
        # the state is that after the first (closed) segment
        M, z = layer.get_state()
        _, M_ref, z_ref = orc.forward(Q[:, :, :N], K[:, :, :N], V[:, :, :N], beta, N, "linear", eps=w.eps)
        gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, gu.tol_for("bf16"))
        layer.decode_flush()
        assert layer.decode_position() == 0
        M, z = layer.get_state()
        _, M_ref, z_ref = orc.forward(Q[:, :, :N + 3], K[:, :, :N + 3], V[:, :, :N + 3], beta, N, "linear",
                                      eps=w.eps)
        gu.check_state(M.cpu().numpy(), z.cpu().numpy(), M_ref, z_ref, gu.tol_for("bf16"))
        # reset drops an open segment; decoding restarts from zero memory
        layer.decode_step(*tok(0))
        layer.reset_state()
        assert layer.decode_position() == 0
        out = layer.decode_step(*tok(0)).float().cpu().numpy()
        ref, _, _, _ = orc.decode_stream(Q[:, :, :1], K[:, :, :1], V[:, :, :1], beta, N, "linear", eps=w.eps)
        gu.check_output(out[:, :, None], ref, gu.tol_for("bf16"))
        with pytest.raises(binding.InfiniAttnError):
            layer.forward_stream(*dev)


def test_full_size_decode_sampled_against_oracle():
    """8 heads, d=128, N=2048: a whole segment and 4 more tokens, token by token; sampled
    tokens against the oracle's decode_token with the cache and state they see."""
    gu.require_gpu()
    base = wl.WORKLOADS[wl.THROUGHPUT_WORKLOAD]
    N = base.segment_len
    L = N + 4
    w = base.with_tokens(L).with_batch(2)
    gu.note(f"[decode] full size: {w.name}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    with binding.InfiniAttention(w.batch, w.heads, w.head_dim, N, update=w.update, eps=w.eps, beta=beta) as layer:
        out = _decode_all(layer, Q, K, V, "bf16", flush=False)
        assert layer.decode_position() == 4
    scale = 1.0 / np.sqrt(w.head_dim)
    tol = gu.tol_for("bf16")
    for b in range(w.batch):
        for h in range(w.heads):
            M0, z0 = np.zeros((w.head_dim, w.head_dim)), np.zeros(w.head_dim)
            M1, z1 = orc.advance(K[b, h, :N], V[b, h, :N], M0, z0, w.update, w.eps)
            for t in (0, 1, 700, N - 1, N, N + 3):
                lo = 0 if t < N else N
                Ms, zs = (M0, z0) if t < N else (M1, z1)
                ref, _, _ = orc.decode_token(Q[b, h, t], K[b, h, t], V[b, h, t], K[b, h, lo:t], V[b, h, lo:t], Ms, zs,
                                             beta[h], w.eps, scale)
                gu.check_output(out[b, h, t][None], ref[None], tol, f"b{b} h{h} t{t}")


def test_split_decode_is_deterministic():
    """One sequence, 2 heads, d=128, a 700-token segment: every token past the 256th splits
    its keys over several workgroups, whose partial states are merged in chunk order by
    whichever finishes last; two runs give the same bits."""
    gu.require_gpu()
    base = wl.WORKLOADS[wl.THROUGHPUT_WORKLOAD]
    N = 700
    w = wl.Workload("decode-split-det", 1, 2, base.head_dim, N, N, "bf16", "linear", seed=53)
    gu.note(f"[decode] split determinism: {w.name}")
    Q, K, V = wl.stream_inputs(w)
    beta = wl.beta_for(w)
    runs = []
    for _ in range(2):
        with binding.InfiniAttention(1, w.heads, w.head_dim, N, update="linear", eps=w.eps, beta=beta) as layer:
            runs.append(_decode_all(layer, Q, K, V, "bf16", flush=False))
    assert np.array_equal(runs[0], runs[1])
    O_ref, _, _, _ = orc.decode_stream(Q, K, V, beta, N, "linear", eps=w.eps)
    gu.check_output(runs[0], O_ref, gu.tol_for("bf16"))
