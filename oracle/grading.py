"""How a GPU result is graded against the oracle -- TEST INFRASTRUCTURE ONLY.

Near-threshold tiles may legitimately be decided either way: the GPU forms
scores in fp32 from bf16 products and compares in the log2 domain, the
oracle in fp64.  A tile is "near" when |exp(delta) / threshold - 1| <= 1e-3,
with delta the oracle's fp64 decision statistic (tile_max - running max, max
over the block's rows, natural-log units as in the skip test of the design
page "Skip-Softmax", section "The skip test").  Every other tile must match
exactly, and overall agreement must be >= 99.9 %.  Outputs are graded
against the oracle re-run with the GPU's own mask forced, so a legitimate
flip is not counted as output error: once over all graded rows (relative
L2) and once per row, so that a few wrong rows cannot hide inside a large
case.

Pinned on the CPU by tests/test_grading_pins.py (hand-built masks and
vectors with known answers) and by planted mistakes in
tests/test_oracle_mutations.py.
"""

from __future__ import annotations

import numpy as np

NEAR_REL = 1e-3
MIN_AGREEMENT = 0.999
# Per-row bound = ROW_FACTOR x the global bound of the path (bf16: 1e-2).
# A bf16 output row carries up to 2^-8 relative rounding of its own and of
# the bf16 P weights, ~3e-3 together; a row that lost or gained a tile's
# worth of softmax mass is off by that mass fraction, usually >> 3 %.
ROW_FACTOR = 3.0


def near_threshold(delta: np.ndarray, thr: float) -> np.ndarray:
    """True where the fp64 statistic ``delta`` (natural log) lies within a
    relative 1e-3 of the threshold: |exp(delta) / thr - 1| <= 1e-3.  With a
    threshold of 0 nothing is near (no tile can pass a strict < 0 test), and
    a non-finite delta (a row block with no visible key, or a first visible
    tile) is never near."""
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
    """||a - b|| / ||b|| over all elements (b is the reference)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_rel_l2(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row relative L2 over the last axis, ||a_r - b_r|| / ||b_r||, b the
    reference.  A reference row whose norm is below 1e-3 of the RMS row norm
    (e.g. a row that sees no key and must be 0) is measured against that
    floor instead, so an all-zero row that the GPU also leaves at 0 grades 0
    and a nonzero one grades large."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    a2 = a.reshape(-1, a.shape[-1])
    b2 = b.reshape(-1, b.shape[-1])
    nb = np.linalg.norm(b2, axis=1)
    rms = float(np.sqrt(np.mean(nb ** 2))) if nb.size else 0.0
    floor = max(1e-3 * rms, 1e-300)
    return np.linalg.norm(a2 - b2, axis=1) / np.maximum(nb, floor)


def max_row_rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    e = row_rel_l2(a, b)
    return float(e.max()) if e.size else 0.0
