"""How a GPU result is graded against the oracle -- TEST INFRASTRUCTURE ONLY.

Near-threshold tiles may legitimately be decided either way: the GPU forms
scores in fp32 from bf16 products and compares in the log2 domain, the
oracle in fp64.  A tile is "near" when |exp(delta) / threshold - 1| <= 1e-3,
with delta the oracle's fp64 decision statistic (tile_max - running max, max
over the block's rows).  Every other tile must match exactly, and overall
agreement must be >= 99.9 %.  Outputs are graded against the oracle re-run
with the GPU's own mask forced, so a legitimate flip is not counted as output
error.
"""

from __future__ import annotations

import numpy as np

NEAR_REL = 1e-3
MIN_AGREEMENT = 0.999


def near_threshold(delta: np.ndarray, thr: float) -> np.ndarray:
    d = np.asarray(delta, dtype=np.float64)
    if thr <= 0:
        return np.zeros(d.shape, bool)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.exp(d) / thr
        near = np.abs(r - 1.0) <= NEAR_REL
    return np.where(np.isfinite(d), near, False)


def grade_masks(gpu_mask: np.ndarray, ref_mask: np.ndarray, ref_delta: np.ndarray,
                thr: float, select=None) -> dict:
    """Compare masks under the margin rule.  ``select``: optional boolean array
    restricting the comparison (e.g. the sampled blocks of a large case)."""
    g = np.asarray(gpu_mask)
    r = np.asarray(ref_mask)
    sel = np.ones(r.shape, bool) if select is None else np.asarray(select, bool)
    near = near_threshold(ref_delta, thr) & sel
    diff = (g != r) & sel
    far_diff = diff & ~near
    n = int(sel.sum())
    agree = 1.0 - (diff.sum() / n if n else 0.0)
    return {"n": n, "mismatch": int(diff.sum()), "far_mismatch": int(far_diff.sum()),
            "near": int(near.sum()), "agreement": float(agree),
            "ok": bool(far_diff.sum() == 0 and agree >= MIN_AGREEMENT)}


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
