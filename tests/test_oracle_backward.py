"""Pins of the backward oracle (CPU only): its forward against the numpy oracle, its
gradients against central finite differences of the numpy oracle (a route that shares
nothing with autograd), and the gate-closed case against PyTorch's own attention
backward.  Planted mistakes in its forward must fail one of these."""

import math

import numpy as np
import pytest
import torch

from oracle import infini_backward as ob
from oracle import infini_oracle as orc


@pytest.fixture
def rng():
    return np.random.default_rng(1234)


def _inputs(rng, B=1, H=2, L=11, d=3, N=4):
    s = 1.2 / math.sqrt(d)
    Q, K, V = (rng.standard_normal((B, H, L, d)) * s for _ in range(3))
    beta = rng.standard_normal(H)
    M0 = rng.standard_normal((B, H, d, d)) * 0.3
    z0 = np.abs(rng.standard_normal((B, H, d))) + 0.5   # a plausible (positive) key sum
    dO = rng.standard_normal((B, H, L, d))
    dM = rng.standard_normal((B, H, d, d)) * 0.2
    dz = rng.standard_normal((B, H, d)) * 0.2
    return Q, K, V, beta, M0, z0, dO, dM, dz, N


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_torch_forward_matches_the_numpy_oracle(rng, update):
    Q, K, V, beta, M0, z0, _, _, _, N = _inputs(rng, B=2, L=13)
    t = lambda x: torch.tensor(x)   # noqa: E731
    O, M, z = ob.forward_torch(t(Q), t(K), t(V), t(beta), N, update, 1e-6, None, t(M0), t(z0))
    O2, M2, z2 = orc.forward(Q, K, V, beta, N, update, eps=1e-6, M0=M0, z0=z0)
    np.testing.assert_allclose(O.numpy(), O2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(M.numpy(), M2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z.numpy(), z2, rtol=1e-13, atol=1e-14)


def _loss_numpy(Q, K, V, beta, M0, z0, dO, dM, dz, N, update):
    O, M, z = orc.forward(Q, K, V, beta, N, update, eps=1e-6, M0=M0, z0=z0)
    return float((O * dO).sum() + (M * dM).sum() + (z * dz).sum())


@pytest.mark.parametrize("update", ["linear", "delta"])
def test_gradients_match_central_differences_of_the_numpy_forward(rng, update):
    Q, K, V, beta, M0, z0, dO, dM, dz, N = _inputs(rng)
    gr = ob.gradients(Q, K, V, beta, dO, N, update, 1e-6, None, M0, z0, dM, dz)
    args = dict(Q=Q, K=K, V=V, beta=beta, M0=M0, z0=z0)
    grad_of = dict(Q="dQ", K="dK", V="dV", beta="dbeta", M0="dM0", z0="dz0")
    h = 1e-5
    for name, x in args.items():
        for trial in range(2):
            delta = rng.standard_normal(np.shape(x))
            plus, minus = dict(args), dict(args)
            plus[name] = x + h * delta
            minus[name] = x - h * delta
            fd = (_loss_numpy(**plus, dO=dO, dM=dM, dz=dz, N=N, update=update) -
                  _loss_numpy(**minus, dO=dO, dM=dM, dz=dz, N=N, update=update)) / (2 * h)
            an = float((gr[grad_of[name]] * delta).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, trial, fd, an)


def test_closed_gate_gives_the_causal_attention_gradient(rng):
    """beta = -inf, no upstream gradient on the state: only the local attention sees dO, so
    dQ, dK, dV are those of causal SDPA inside each segment, and dbeta = 0."""
    Q, K, V, _, _, _, dO, _, _, N = _inputs(rng, B=2, H=2, L=10, d=4, N=4)
    gr = ob.gradients(Q, K, V, np.full(2, -np.inf), dO, N, "delta")
    assert np.all(gr["dbeta"] == 0)
    for lo in range(0, 10, N):
        hi = min(lo + N, 10)
        q, k, v = (torch.tensor(x[:, :, lo:hi], requires_grad=True) for x in (Q, K, V))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.5)
        dq, dk, dv = torch.autograd.grad((o * torch.tensor(dO[:, :, lo:hi])).sum(), [q, k, v])
        np.testing.assert_allclose(gr["dQ"][:, :, lo:hi], dq.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gr["dK"][:, :, lo:hi], dk.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gr["dV"][:, :, lo:hi], dv.numpy(), rtol=1e-10, atol=1e-12)


def test_linear_memory_gradient_closed_form(rng):
    """beta = +inf (memory only), linear rule, zero start, two segments: the first segment
    reads zero memory, so its Q gets no gradient; the second reads M_0 = sigma(K_0)^T V_0,
    so dV_0 = sigma(K_0) sum_t u_t^T dO_t / den_t with u = sigma(Q_1)."""
    d, N = 3, 4
    Q, K, V, _, _, _, dO, _, _, _ = _inputs(rng, B=1, H=1, L=2 * N, d=d, N=N)
    gr = ob.gradients(Q, K, V, np.array([np.inf]), dO, N, "linear")
    assert np.allclose(gr["dQ"][0, 0, :N], 0)
    sk0 = orc.elu_plus_one(K[0, 0, :N])
    u = orc.elu_plus_one(Q[0, 0, N:])
    den = u @ sk0.sum(axis=0) + 1e-6
    dnum = dO[0, 0, N:] / den[:, None]
    # A_mem = u M / den: dL/dM = u^T dnum - u^T ((dO * A_mem).sum(1) / den); M = sk0^T V_0
    a_mem = (u @ (sk0.T @ V[0, 0, :N])) / den[:, None]
    dM = u.T @ dnum
    dz = -u.T @ ((dO[0, 0, N:] * a_mem).sum(axis=1) / den)
    np.testing.assert_allclose(gr["dV"][0, 0, :N], sk0 @ dM, rtol=1e-10, atol=1e-12)
    dsk0 = V[0, 0, :N] @ dM.T + dz[None, :]
    dk0 = dsk0 * np.where(K[0, 0, :N] > 0, 1.0, np.exp(np.minimum(K[0, 0, :N], 0)))
    np.testing.assert_allclose(gr["dK"][0, 0, :N], dk0, rtol=1e-10, atol=1e-12)


def _sigma_without_one(x):
    return torch.where(x > 0, x, torch.exp(torch.clamp(x, max=0.0)) - 1.0)


def _gate_flipped(beta):
    return torch.sigmoid(-beta)


@pytest.mark.parametrize("attr,fn", [("_sigma", _sigma_without_one), ("_gate_value", _gate_flipped)],
                         ids=["sigma-without-one", "gate-flipped"])
def test_a_planted_mistake_in_the_torch_forward_fails_a_pin(monkeypatch, attr, fn):
    monkeypatch.setattr(ob, attr, fn)
    with pytest.raises(AssertionError):
        test_torch_forward_matches_the_numpy_oracle(np.random.default_rng(7), "linear")
