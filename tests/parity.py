"""Comparison rules between the GPU outputs and the fp64 oracle.

* R2 (bf16): |gpu - ref| <= one bf16 ulp of ref, ulp(v) = 2^(floor(log2|v|) - 7)
  (2^-133 below the normal range): either bf16 neighbour of the exact value passes.
* rrms (fp32): |gpu - ref| <= 1e-5 |ref|.
* inj_next, x (bf16): |gpu - ref| <= 2e-2 max|ref| + 2e-2 |ref| (max over the
  compared tensor).
"""
from __future__ import annotations

import numpy as np
import torch

RRMS_RTOL = 1e-5
ATOL_FRAC = 2e-2
RTOL = 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.exp2(e - 7)
    return np.where(a >= 2.0 ** -126, u, 2.0 ** -133)


def check_r2(gpu, ref, what="R2"):
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    err = np.abs(g - ref)
    lim = ulp_bf16(ref)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1 bf16 ulp; worst ratio "
                           f"{float((err / lim).max()):.3f} at {np.unravel_index(np.argmax(err / lim), err.shape)}")


def check_rrms(gpu, ref, what="rrms"):
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    rel = np.abs(g - ref) / np.abs(ref)
    assert float(rel.max()) <= RRMS_RTOL, f"{what}: max relative error {float(rel.max()):.3e} > {RRMS_RTOL}"


def check_tol(gpu, ref, what):
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - ref)
    lim = ATOL_FRAC * float(np.abs(ref).max()) + RTOL * np.abs(ref)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} beyond tolerance; max err {float(err.max()):.4e}, "
                           f"max|ref| {float(np.abs(ref).max()):.4e}")
    return float(err.max()), float(np.abs(ref).max())


def check_all(out: dict, ref: dict, rows=None):
    """out: GPU tensors (R2, rrms, inj_next, x); ref: oracle arrays for ``rows``
    (all rows when None)."""
    sel = (lambda t: t) if rows is None else (lambda t: t[rows])
    check_r2(sel(out["R2"]), ref["R2"])
    check_rrms(sel(out["rrms"]), ref["rrms"])
    check_tol(sel(out["inj_next"]), ref["inj_next"], "inj_next")
    check_tol(sel(out["x"]), ref["x"], "x")
