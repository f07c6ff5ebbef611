"""The allocation-free forward call (infini_attn_forward_stream_noalloc), for callers that
cannot allocate device memory, through the C-ABI against the call it mirrors,
infini_attn_forward_stream: two calls in a row on one handle (the state carried from the
first to the second), the second with a smaller input, under the tolerances of the
oracle parity tests (output max-abs <= 2e-2 and relative <= 1e-2, state within 1e-4), and
bit for bit where both calls use the same window length.  Its window workspace lives in
one static device array shared by every call on the device, which keeps the last call's
contents: the second call must not be disturbed by what the first left there."""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _two_calls(B, H, d, N, L1, L2, update, max_window, seed):
    w1 = wl.Workload(f"noalloc-a-{update}", B, H, d, N, L1, "bf16", update, seed=seed)
    w2 = wl.Workload(f"noalloc-b-{update}", B, H, d, N, L2, "bf16", update, seed=seed + 1)
    beta = wl.beta_for(w1)
    ins = [[gu.to_dev(x, "bf16") for x in wl.stream_inputs(w)] for w in (w1, w2)]
    res = {}
    for mode in ("stream", "noalloc"):
        with binding.InfiniAttention(B, H, d, N, update=update, eps=w1.eps, beta=beta,
                                     max_window_segments=max_window) as layer:
            call = layer.forward_stream if mode == "stream" else layer.forward_stream_noalloc
            outs = []
            for q, k, v in ins:
                out = torch.empty_like(q)
                call(q, k, v, out=out)
                outs.append(out)
            M, z = layer.get_state()
            torch.cuda.synchronize()
            res[mode] = dict(outs=[o.float().cpu().numpy() for o in outs], M=M.cpu().numpy(), z=z.cpu().numpy())
    return res


@pytest.mark.parametrize("update", ["linear", "delta"])
@pytest.mark.parametrize("shape", [(1, 8, 128, 2048, 16 * 2048, 3 * 2048 + 500, 0),
                                   (1, 8, 128, 2048, 16 * 2048, 3 * 2048 + 500, 2),
                                   (2, 2, 64, 256, 5 * 256 + 77, 256 + 3, 0)],
                         ids=["h8-d128-32k-then-6.6k", "h8-d128-window2", "b2-h2-d64-ragged"])
def test_noalloc_matches_forward_stream(update, shape):
    gu.require_gpu()
    B, H, d, N, L1, L2, max_window = shape
    gu.note(f"[noalloc] {update}: B={B} H={H} d={d} N={N} calls of {L1} then {L2} tokens, max window {max_window}")
    res = _two_calls(B, H, d, N, L1, L2, update, max_window, seed=81)
    a, b = res["stream"], res["noalloc"]
    tol = gu.BF16_TOL
    for i in range(2):
        gu.check_output(b["outs"][i], a["outs"][i], tol, what=f"call {i + 1} out")
    gu.check_state(b["M"], b["z"], a["M"].astype(np.float64), a["z"].astype(np.float64), tol)
    same = all(np.array_equal(x, y) for x, y in zip(a["outs"], b["outs"])) and np.array_equal(a["M"], b["M"])
    gu.note(f"  bit-identical: {same}")
    if max_window == 2:   # both calls cut the stream into the same two-segment windows
        assert same, "same windows must give bit-identical results"


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    """512 (batch, head) pairs at d = 128 under the delta rule need ~115 MB of window
    workspace for one segment: more than the 32 MiB array.  The call returns
    INFINI_ERR_SCRATCH before enqueuing anything and leaves the state alone."""
    gu.require_gpu()
    B, H, d, N = 64, 8, 128, 64
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    with binding.InfiniAttention(B, H, d, N, update="delta") as layer:
        with pytest.raises(binding.InfiniAttnError) as ei:
            layer.forward_stream_noalloc(q, q, q, out=torch.empty_like(q))
        assert ei.value.status == binding.ERR_SCRATCH
        M, z = layer.get_state()
        torch.cuda.synchronize()
        assert not M.any() and not z.any()
