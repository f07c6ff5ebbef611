"""Shared helpers of the GPU tests: tolerances, metrics and oracle comparisons.

Tolerances (written here once, used by every GPU parity test):
* bf16 I/O: output max-abs <= 2e-2 and relative (Frobenius) <= 1e-2, globally and per
  (batch, head); the retrieval term A_mem and the local term A_dot each within 1e-2
  relative of their own norm; state M within 1e-4 relative per (batch, head) and z within
  1e-4 relative per entry.
* f32 I/O: the same quantities within 2e-5 (the all-fp32 path).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

BF16_TOL = dict(out_abs=2e-2, out_rel=1e-2, part_rel=1e-2, m_rel=1e-4, z_rel=1e-4)
F32_TOL = dict(out_abs=2e-5, out_rel=2e-5, part_rel=2e-5, m_rel=2e-5, z_rel=2e-5)


def tol_for(io_dtype: str):
    return BF16_TOL if io_dtype == "bf16" else F32_TOL


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, io_dtype: str) -> torch.Tensor:
    dt = torch.bfloat16 if io_dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt).contiguous()


def rel(a, b) -> float:
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def check_output(o, ref, tol, what="out"):
    """o, ref: [..., T, d] arrays; global and per-leading-index checks."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite values"
    err = float(np.abs(o - ref).max())
    r = rel(o, ref)
    assert err <= tol["out_abs"], f"{what}: max-abs {err:.3e} > {tol['out_abs']}"
    assert r <= tol["out_rel"], f"{what}: rel {r:.3e} > {tol['out_rel']}"
    lead = o.reshape(-1, *o.shape[-2:])
    lref = ref.reshape(-1, *ref.shape[-2:])
    for i in range(lead.shape[0]):
        ri = rel(lead[i], lref[i])
        assert ri <= tol["out_rel"], f"{what}[{i}]: rel {ri:.3e}"
    return err, r


def check_part(x, ref, tol, what):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if np.all(ref == 0):
        assert np.all(x == 0), f"{what}: expected exact zeros"
        return 0.0
    r = rel(x, ref)
    assert r <= tol["part_rel"], f"{what}: rel {r:.3e} > {tol['part_rel']}"
    return r


def check_state(M, z, M_ref, z_ref, tol):
    M = np.asarray(M, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    worst_m = 0.0
    lead = M.reshape(-1, *M.shape[-2:])
    lref = M_ref.reshape(-1, *M_ref.shape[-2:])
    for i in range(lead.shape[0]):
        r = rel(lead[i], lref[i])
        worst_m = max(worst_m, r)
    assert worst_m <= tol["m_rel"], f"M: rel {worst_m:.3e} > {tol['m_rel']}"
    zr = float(np.max(np.abs(z - z_ref) / np.abs(z_ref))) if np.all(z_ref != 0) else rel(z, z_ref)
    assert zr <= tol["z_rel"], f"z: rel {zr:.3e} > {tol['z_rel']}"
    return worst_m, zr
