"""Closed forms for the operating point of skip-softmax attention.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py for who may use it).

Source: the vLLM-Omni design page "Skip-Softmax", sections "The threshold"
and "Timestep gating", and the BLASST summary page, section "Calibratie en
Thresholding" (threshold inversely proportional to the context length).
"""

from __future__ import annotations

import math


def factor_calibrated(a: float, b: float, target_sparsity: float) -> float:
    """Calibrated factor: a * exp(b * target_sparsity), a and b fitted per model."""
    return a * math.exp(b * target_sparsity)


def factor_direct(threshold: float, seqlen: int) -> float:
    """Calibration-free factor: the user threshold times the sequence length."""
    return threshold * seqlen


def threshold(factor: float, seqlen: int) -> float:
    """Per-tile threshold normalised by the sequence length: factor / seqlen."""
    return factor / seqlen


def gate_enabled(timestep: float | None, disabled_until: float | None) -> bool:
    """Whether the sparse mode is on at normalised timestep ``timestep``.

    Unset ``disabled_until``: always on.  Set, but no timestep published:
    dense.  Otherwise on once t <= disabled_until (t runs from 1.0 down to 0.0).
    """
    if disabled_until is None:
        return True
    if timestep is None:
        return False
    return timestep <= disabled_until
