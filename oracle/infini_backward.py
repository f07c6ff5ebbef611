"""Gradients of the Infini-attention layer forward: the CPU oracle of the backward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  The GPU library never
calls it and shares no code with it.

What it is: the layer forward of ``oracle.infini_oracle`` restated with plain PyTorch
float64 CPU operations (same order of steps: read the memory with the previous state,
local causal attention, gate, then write the memory; segment by segment, every (batch,
head) chain independent), and its gradients taken by ``torch.autograd`` -- the exact
derivative of that definition, back through the whole M / z recurrence
(backpropagation through time over the segments, section "Training Infrastructure for
Recurrent Attention" of the architecture summary of arXiv 2404.07143).

Inputs of the gradient: Q, K, V [B, H, L, d], the gate logits beta [H], the initial state
M0 [B, H, d, d], z0 [B, H, d]; the upstream gradient dO of the output [B, H, L, d] and,
optionally, dM and dz of the final state.  The same readings as the forward oracle apply
(eps in both retrieval denominators, ELU alpha = 1, one beta per head, the delta rule's
retrieved value from the state before the segment).
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["forward_torch", "gradients"]


def _sigma(x):
    # ELU + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise
    return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))


def _gate_value(beta):
    return torch.sigmoid(beta)


def forward_torch(Q, K, V, beta, segment_len, update="linear", eps=1e-6, scale=None, M0=None, z0=None):
    """The layer over a stream in torch float64 (differentiable).  Returns (O, M, z)."""
    B, H, L, d = Q.shape
    dv = V.shape[-1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    M = torch.zeros((B, H, d, dv), dtype=torch.float64) if M0 is None else M0
    z = torch.zeros((B, H, d), dtype=torch.float64) if z0 is None else z0
    g = _gate_value(beta).reshape(1, H, 1, 1)
    outs = []
    for lo in range(0, L, segment_len):
        hi = min(lo + segment_len, L)
        q, k, v = Q[:, :, lo:hi], K[:, :, lo:hi], V[:, :, lo:hi]
        n = hi - lo
        # memory read with the state before the segment (Eq. 7)
        sq = _sigma(q)
        a_mem = (sq @ M) / ((sq @ z.unsqueeze(-1)) + eps)
        # local causal attention (Eq. 6)
        s = scale * (q @ k.transpose(-1, -2))
        future = torch.triu(torch.ones((n, n), dtype=torch.bool), diagonal=1)
        s = s.masked_fill(future, float("-inf"))
        a_dot = torch.softmax(s, dim=-1) @ v
        # gate (Eq. 10)
        outs.append(g * a_mem + (1.0 - g) * a_dot)
        # memory write (Eq. 8 / Eq. 9)
        sk = _sigma(k)
        if update == "linear":
            M = M + sk.transpose(-1, -2) @ v
        elif update == "delta":
            retrieved = (sk @ M) / ((sk @ z.unsqueeze(-1)) + eps)
            M = M + sk.transpose(-1, -2) @ (v - retrieved)
        else:
            raise ValueError(f"unknown update rule {update!r}")
        z = z + sk.sum(dim=-2)
    return torch.cat(outs, dim=2), M, z


def gradients(Q, K, V, beta, dO, segment_len, update="linear", eps=1e-6, scale=None, M0=None, z0=None,
              dM=None, dz=None):
    """d(loss)/d(Q, K, V, beta, M0, z0) for loss = <dO, O> + <dM, M_final> + <dz, z_final>.

    Returns a dict of float64 numpy arrays: dQ, dK, dV [B, H, L, d], dbeta [H],
    dM0 [B, H, d, d], dz0 [B, H, d]; plus O, M, z of the forward.
    """
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)   # noqa: E731
    B, H, L, d = np.shape(Q)
    Qt, Kt, Vt, bt = t(Q), t(K), t(V), t(np.asarray(beta, dtype=np.float64).reshape(H))
    Mt = t(np.zeros((B, H, d, np.shape(V)[-1])) if M0 is None else M0)
    zt = t(np.zeros((B, H, d)) if z0 is None else z0)
    O, M, z = forward_torch(Qt, Kt, Vt, bt, segment_len, update, eps, scale, Mt, zt)
    loss = (O * torch.tensor(np.asarray(dO, dtype=np.float64))).sum()
    if dM is not None:
        loss = loss + (M * torch.tensor(np.asarray(dM, dtype=np.float64))).sum()
    if dz is not None:
        loss = loss + (z * torch.tensor(np.asarray(dz, dtype=np.float64))).sum()
    grads = torch.autograd.grad(loss, [Qt, Kt, Vt, bt, Mt, zt])
    names = ["dQ", "dK", "dV", "dbeta", "dM0", "dz0"]
    out = {n: g_.detach().numpy() for n, g_ in zip(names, grads)}
    out.update(O=O.detach().numpy(), M=M.detach().numpy(), z=z.detach().numpy())
    return out
