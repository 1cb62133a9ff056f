"""Comparison helpers for the GPU parity tests.

Tolerances for floating-point outputs of bf16/fp8 inputs: max-abs 2e-2 and
rel_l2 1e-2 against the fp64 oracle fed the same quantised values; LayerNorm
statistics within 1e-5 (rstd relative; mean relative to sqrt(var + eps)),
evaluated by running the oracle LayerNorm on the GPU's own fp32 residual
stream so that the attention error does not leak into the statistics check.
"""
from __future__ import annotations

import numpy as np
import torch

MAX_ABS = 2e-2
REL_L2 = 1e-2
# The worst single row (last dimension: a head's D outputs, or a hidden row)
# must also stay within 3x the whole-tensor bound: over tens of thousands of
# rows one wrong row barely moves the whole-tensor rel_l2, while its own
# rel_l2 is of order 1.  Rows whose reference is all zero (fully masked
# queries) are held to MAX_ABS by the element check instead.
ROW_REL_L2 = 3e-2
LN_STAT = 1e-5
# log-sum-exp outputs: the kernels normalise by the sum of the bf16-rounded
# probabilities they multiply into V (each within 2^-9 relative of the exact
# one), so |delta lse| <= ln(1 + 2^-9) + fp32 rounding; allow 2^-8.
LSE_ABS = 2.0 ** -8


def to64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().double().numpy() if x.dtype != torch.float64 else x.cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_l2_max(got, ref) -> float:
    """Largest rel_l2 of one row (rows along the reference's last dimension)
    among the rows whose reference is not all zero."""
    g64, r64 = to64(got), to64(ref)
    if r64.ndim < 2 or r64.size == 0:
        return 0.0
    n = r64.shape[-1]
    g, r = g64.reshape(-1, n), r64.reshape(-1, n)
    dn = np.linalg.norm(g - r, axis=1)
    rn = np.linalg.norm(r, axis=1)
    live = rn > 0
    return float(np.max(dn[live] / rn[live])) if np.any(live) else 0.0


def metrics(got, ref) -> dict:
    g, r = to64(got).ravel(), to64(ref).ravel()
    d = g - r
    nr = np.linalg.norm(r)
    return {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rel_l2": float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
        "row_rel_l2_max": row_rel_l2_max(got, ref) if np.all(np.isfinite(g)) else float("inf"),
        "cos": float(g @ r / (np.linalg.norm(g) * nr)) if nr > 0 and np.linalg.norm(g) > 0 else 1.0,
        "finite": bool(np.all(np.isfinite(g))),
    }


def assert_close(got, ref, what: str, max_abs: float = MAX_ABS, rel_l2: float = REL_L2,
                 row_rel_l2: float = ROW_REL_L2) -> dict:
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite values {m}"
    assert m["max_abs"] <= max_abs and m["rel_l2"] <= rel_l2, f"{what}: {m}"
    assert m["row_rel_l2_max"] <= row_rel_l2, f"{what}: worst row {m}"
    return m


def assert_ln_stats(res_out_gpu, mean_gpu, rstd_gpu, gamma, beta, eps, what: str):
    import oracle

    x = to64(res_out_gpu)
    _, mu, rs = oracle.layernorm(x, None, None, eps)
    mg, rg = to64(mean_gpu).ravel(), to64(rstd_gpu).ravel()
    sd = 1.0 / rs  # sqrt(var + eps)
    e_mean = float(np.max(np.abs(mg - mu) / sd))
    e_rstd = float(np.max(np.abs(rg - rs) / rs))
    assert e_mean <= LN_STAT and e_rstd <= LN_STAT, f"{what}: mean err {e_mean:.3g}, rstd err {e_rstd:.3g}"
    return e_mean, e_rstd
