"""GPU checks of the delta rule's fixed point (invariant 4 of the oracle's pins): writing a
key / value pair that the memory already retrieves exactly leaves M unchanged, while z
still grows (architecture summary of arXiv 2404.07143, section 3.4 "Compressive Memory:
The Recurrent Long-Range Arm", the delta-rule paragraph under Eq. 9: the update adds only
the part of V that retrieval does not already return; z advances as in Eq. 8).

One segment of n copies of the same (k, v) written into the zero memory gives
M_1 = n sigma(k)^T v and z_1 = n sigma(k) (segment 0 retrieves 0, so the delta write equals
the linear one).  Writing the same segment again retrieves
R = sigma(k) M_1 / (sigma(k) z_1 + eps) = v (1 - eps / (n |sigma(k)|^2 + eps)), so
M_2 - M_1 = n sigma(k)^T (v - R) is below 1e-11 of |M_1| in exact arithmetic: the GPU's
M - G M + U form must cancel to the state tolerance, ||M_2 - M_1|| / ||M_1|| <= 1e-4, and
z_2 - z_1 = n sigma(k) to 1e-4.  Checked through each way the state advances: two calls of
forward_stream, two calls of forward_segment, and one forward_stream call over both
segments (the chain inside one window), at the full segment length of the throughput
workloads (d = 128, N = 2048) and on a short ragged segment (d = 64, n = 300 < N).
"""

import numpy as np
import pytest
import torch

from compressive_memory_transformer_segment_amd import binding
from compressive_memory_transformer_segment_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-4


def _sigma64(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _pair_segment(B, H, d, n, seed):
    """Q random; K and V: n copies of one (k, v) per (batch, head), bf16-rounded."""
    rng = np.random.default_rng(seed)
    k = wl.round_to_bf16((rng.standard_normal((B, H, 1, d)) / np.sqrt(d)).astype(np.float32))
    v = wl.round_to_bf16((rng.standard_normal((B, H, 1, d)) / np.sqrt(d)).astype(np.float32))
    q = wl.round_to_bf16((rng.standard_normal((B, H, n, d)) / np.sqrt(d)).astype(np.float32))
    K = np.ascontiguousarray(np.broadcast_to(k, (B, H, n, d)))
    V = np.ascontiguousarray(np.broadcast_to(v, (B, H, n, d)))
    return q, K, V, k[:, :, 0], v[:, :, 0]


def _rel_per_head(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1, *np.shape(a)[-2:])
    b = np.asarray(b, dtype=np.float64).reshape(-1, *np.shape(b)[-2:])
    return max(gu.rel(a[i], b[i]) for i in range(a.shape[0]))


@pytest.mark.parametrize("path", ["stream-calls", "segment-calls", "one-stream-call"])
@pytest.mark.parametrize("shape", [(1, 2, 128, 2048, 2048), (2, 1, 64, 2048, 300)],
                         ids=["d128-n2048", "d64-n300-ragged"])
def test_delta_rewrite_of_a_retrievable_pair_keeps_memory(path, shape):
    gu.require_gpu()
    B, H, d, N, n = shape
    gu.note(f"[invariant 4] delta rewrite, {path}: B={B} H={H} d={d} N={N} n={n}")
    Q, K, V, k, v = _pair_segment(B, H, d, n, seed=71 + d + n)
    sk = _sigma64(k)                                    # [B, H, d]
    M1_ref = n * sk[..., :, None] * v.astype(np.float64)[..., None, :]
    z1_ref = n * sk
    dev = [gu.to_dev(x, "bf16") for x in (Q, K, V)]
    seg = n if path == "one-stream-call" else N   # one call over two segments of n tokens
    with binding.InfiniAttention(B, H, d, seg, update="delta", eps=1e-6, beta=[0.0] * H) as layer:
        if path == "one-stream-call":
            out = layer.forward_stream(*(torch.cat([x, x], dim=2).contiguous() for x in dev))
            M2, z2 = layer.get_state()
            torch.cuda.synchronize()
            M1, z1 = M1_ref, z1_ref
        else:
            call = layer.forward_stream if path == "stream-calls" else layer.forward_segment
            call(*dev)
            M1, z1 = (x.cpu().numpy() for x in layer.get_state())
            out = call(*dev)
            M2, z2 = layer.get_state()
            torch.cuda.synchronize()
        M2, z2 = M2.cpu().numpy(), z2.cpu().numpy()
        assert torch.isfinite(out.float()).all()
    r1 = _rel_per_head(M1, M1_ref)
    r21 = _rel_per_head(M2, M1)
    dz = np.asarray(z2, dtype=np.float64) - np.asarray(z1, dtype=np.float64)
    zr = float(np.max(np.abs(dz - z1_ref) / z1_ref))
    gu.note(f"  ||M1 - n s(k)^T v|| / ||.|| = {r1:.2e}, ||M2 - M1|| / ||M1|| = {r21:.2e}, z growth rel {zr:.2e}")
    assert r1 <= STATE_TOL, f"M after the first write: rel {r1:.3e}"
    assert r21 <= STATE_TOL, f"rewrite changed M: rel {r21:.3e} > {STATE_TOL}"
    assert zr <= STATE_TOL, f"z growth: rel {zr:.3e}"
