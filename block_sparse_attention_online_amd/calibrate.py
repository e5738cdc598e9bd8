"""Calibration of the skip threshold on the kernels themselves.

The design page "Skip-Softmax" (section "The threshold") fits a and b of the
calibrated factor a*exp(b*target_sparsity) per model so that a target
sparsity lands near that fraction of skipped tiles; the BLASST summary page
(section "Calibratie en Thresholding") describes an automated procedure that
picks the constant so a fixed sparsity (e.g. 70 %) holds at every context
length, with threshold = a / L.

The pages give no procedure beyond that, so this module takes the plainest
one: skipped-tile fraction is non-decreasing in the threshold (the test is
exp(tile_max - running_max) < threshold with everything else fixed), so a
bisection in log(threshold) on the kernel's own skip mask finds the threshold
for a target; (a, b) then come from a least-squares line through
ln(threshold * L) = ln a + b * s over measured (threshold, L, s) points.

A fitted line may ask for more than the test can mean: above a threshold of
1 the test exp(tile_max - running_max) < threshold no longer bounds a skipped
key's softmax weight (it passes tiles whose maximum exceeds the running
max), so a calibrated threshold is clamped to 1 and the target reported as
not reachable there, exactly as bisection reports a target that even a
threshold of 1 does not reach.
"""

from __future__ import annotations

import math

import torch


def skip_fraction(mask: torch.Tensor) -> float:
    """Skipped / visited tiles of a kernel skip mask (0 kept, 1 skipped, 2 not visited)."""
    sk = int((mask == 1).sum().item())
    vis = sk + int((mask == 0).sum().item())
    return sk / vis if vis else 0.0


def bisect_threshold(run, target: float, lo: float = 1e-8, hi: float = 1.0,
                     iters: int = 30, tol: float = 0.005) -> tuple:
    """Threshold in [lo, hi] whose skip fraction ``run(thr)`` is closest to ``target``.

    Returns (threshold, achieved skip, reachable) -- reachable is False when
    even ``hi`` skips less than the target."""
    s_hi = run(hi)
    if s_hi < target - tol:
        return hi, s_hi, False
    s_lo = run(lo)
    if s_lo >= target - tol:
        return lo, s_lo, True
    best = (hi, s_hi)
    a, b = math.log(lo), math.log(hi)
    for _ in range(iters):
        mid = 0.5 * (a + b)
        thr = math.exp(mid)
        s = run(thr)
        if abs(s - target) < abs(best[1] - target):
            best = (thr, s)
        if abs(s - target) <= tol:
            break
        if s < target:
            a = mid
        else:
            b = mid
    return best[0], best[1], True


def calibrated_threshold(a: float, b: float, target: float, seqlen: int, *,
                         timestep=None, disabled_until=None) -> tuple:
    """(threshold, reachable) for the calibrated factor a*exp(b*target) / seqlen
    as the library resolves it (timestep gating included: 0 when gated off),
    clamped to at most 1.  ``reachable`` is False when the fit asked for a
    threshold above 1."""
    from . import ss_resolve_threshold

    thr = ss_resolve_threshold("calibrated", a=a, b=b, target_sparsity=target, seqlen=seqlen,
                               timestep=timestep, disabled_until=disabled_until)
    if thr > 1.0:
        return 1.0, False
    return thr, True


def fit_factor(points) -> tuple:
    """Least-squares (a, b) of ln(threshold * L) = ln a + b * s over
    ``points`` = [(threshold, L, s), ...].  With a single distinct s, b = 0.
    The line is not bounded: use calibrated_threshold to turn it into a
    threshold a kernel call may take."""
    xs = [p[2] for p in points]
    ys = [math.log(p[0] * p[1]) for p in points]
    n = len(points)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    b = 0.0 if sxx == 0 else sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    return math.exp(my - b * mx), b
