"""Pins of the grader that decides every GPU parity verdict (CPU only).

The rule graded here is the one the skip test implies (design page
"Skip-Softmax", section "The skip test": a tile is skipped when
exp(tile_max - running_max) is strictly below the threshold): a tile whose
fp64 statistic sits within a relative 1e-3 of the threshold may fall either
way on hardware that rounds differently, every other tile must match, and
at least 99.9 % of the graded tiles must agree.  Every expected value below
is worked out by hand from that rule; none comes from a GPU.
"""

import math

import numpy as np
import pytest

from oracle import grading


# --------------------------------------------------------------------------- near_threshold

@pytest.mark.parametrize("thr", [1e-4, 0.01, 0.7105, 1.0, 3.0])
def test_near_band_is_relative_one_in_a_thousand_in_natural_log_units(thr):
    ln = math.log(thr)
    inside = [ln, math.log(thr * (1 + 0.9e-3)), math.log(thr * (1 - 0.9e-3))]
    outside = [math.log(thr * (1 + 1.1e-3)), math.log(thr * (1 - 1.1e-3)),
               math.log(thr * 1.05), math.log(thr * 0.95), ln + 1.0, ln - 1.0]
    if abs(ln) > 0.01:
        outside.append(ln / math.log(2.0))  # the same number read in log2 units is far away
    got = grading.near_threshold(np.array(inside + outside), thr)
    assert got.tolist() == [True] * len(inside) + [False] * len(outside)


def test_nothing_is_near_a_zero_threshold():
    d = np.array([-math.inf, -50.0, -1e-9, 0.0, 1.0, math.inf])
    assert not grading.near_threshold(d, 0.0).any()


def test_non_finite_statistics_are_never_near():
    # -inf: a row block with no visible key votes skip; +inf: a first visible
    # tile; nan must not count either.
    d = np.array([-math.inf, math.inf, math.nan])
    for thr in (1e-3, 1.0, 5.0):
        assert not grading.near_threshold(d, thr).any()


def test_near_keeps_the_shape():
    d = np.full((2, 3, 4), math.log(0.2))
    assert grading.near_threshold(d, 0.2).shape == (2, 3, 4)
    assert grading.near_threshold(d, 0.2).all()


# --------------------------------------------------------------------------- grade_masks

def _case(n=10000, thr=0.01, seed=0):
    """A mask and statistics where every tile is far from the threshold
    (|delta - ln thr| >= 0.5), the mask being the rule applied to delta."""
    rng = np.random.default_rng(seed)
    off = rng.uniform(0.5, 3.0, n) * rng.choice([-1.0, 1.0], n)
    delta = math.log(thr) + off
    mask = (delta < math.log(thr)).astype(np.uint8)
    return mask, delta


def test_identical_masks_pass_with_full_agreement():
    mask, delta = _case()
    g = grading.grade_masks(mask.copy(), mask, delta, 0.01)
    assert g == {"n": 10000, "mismatch": 0, "far_mismatch": 0, "near": 0,
                 "agreement": 1.0, "ok": True}


def test_one_far_flip_fails_even_at_high_agreement():
    mask, delta = _case()
    gpu = mask.copy()
    gpu[1234] ^= 1
    g = grading.grade_masks(gpu, mask, delta, 0.01)
    assert g["mismatch"] == 1 and g["far_mismatch"] == 1
    assert g["agreement"] == pytest.approx(0.9999)
    assert not g["ok"]


def test_one_near_flip_passes():
    mask, delta = _case()
    delta[77] = math.log(0.01 * (1 + 4e-4))
    mask[77] = 0
    gpu = mask.copy()
    gpu[77] = 1
    g = grading.grade_masks(gpu, mask, delta, 0.01)
    assert g["near"] == 1 and g["mismatch"] == 1 and g["far_mismatch"] == 0
    assert g["ok"]


@pytest.mark.parametrize("flips,ok", [(10, True), (11, False), (20, False)])
def test_near_flips_above_one_in_a_thousand_fail(flips, ok):
    mask, delta = _case()
    idx = np.arange(flips) * 7
    delta[idx] = math.log(0.01)
    mask[idx] = 0
    gpu = mask.copy()
    gpu[idx] = 1
    g = grading.grade_masks(gpu, mask, delta, 0.01)
    assert g["far_mismatch"] == 0 and g["mismatch"] == flips
    assert g["agreement"] == pytest.approx(1 - flips / 10000)
    assert g["ok"] is ok


def test_unselected_tiles_are_ignored_and_not_counted():
    mask, delta = _case(n=100)
    gpu = mask.copy()
    gpu[:10] ^= 1          # far flips, all outside the selection
    sel = np.zeros(100, bool)
    sel[10:60] = True
    g = grading.grade_masks(gpu, mask, delta, 0.01, select=sel)
    assert g["n"] == 50 and g["mismatch"] == 0 and g["ok"]
    sel[5] = True          # now one far flip is selected
    g = grading.grade_masks(gpu, mask, delta, 0.01, select=sel)
    assert g["n"] == 51 and g["far_mismatch"] == 1 and not g["ok"]


def test_any_flip_at_zero_threshold_fails():
    mask = np.zeros(5000, np.uint8)
    delta = np.full(5000, -40.0)   # exp(delta) ~ 4e-18: far below any positive threshold
    gpu = mask.copy()
    gpu[3] = 1
    assert not grading.grade_masks(gpu, mask, delta, 0.0)["ok"]


def test_unvisited_code_must_match_too():
    # 2 = not visited (causal upper triangle); a kernel that wrote 0 there is wrong
    mask = np.array([[0, 1, 2, 2]] * 1000, np.uint8)
    delta = np.array([[math.inf, -5.0, -math.inf, -math.inf]] * 1000)
    gpu = mask.copy()
    gpu[17, 3] = 0
    assert not grading.grade_masks(gpu, mask, delta, 0.1)["ok"]


# --------------------------------------------------------------------------- rel_l2 and row errors

def test_rel_l2_literal_values():
    assert grading.rel_l2([1.0, 2.0, 2.0], [0.0, 0.0, 3.0]) == pytest.approx(math.sqrt(6) / 3)
    b = np.array([3.0, -4.0, 12.0])
    assert grading.rel_l2(2 * b, b) == pytest.approx(1.0)
    assert grading.rel_l2(b, 2 * b) == pytest.approx(0.5)   # the reference is the second operand
    assert grading.rel_l2(b, b) == 0.0


def test_row_errors_literal_values():
    a = np.array([[1.0, 0.0], [0.0, 0.0], [3.0, 4.0]])
    b = np.array([[2.0, 0.0], [0.0, 0.0], [3.0, 0.0]])
    e = grading.row_rel_l2(a, b)
    assert e.tolist() == pytest.approx([0.5, 0.0, 4.0 / 3.0])
    assert grading.max_row_rel_l2(a, b) == pytest.approx(4.0 / 3.0)
    # a row that must be zero but is not: measured against 1e-3 of the RMS row norm
    a[1] = [0.01, 0.0]
    rms = math.sqrt((4.0 + 0.0 + 9.0) / 3)
    assert grading.row_rel_l2(a, b)[1] == pytest.approx(0.01 / (1e-3 * rms))


def test_row_errors_keep_leading_axes():
    rng = np.random.default_rng(1)
    b = rng.standard_normal((2, 3, 5, 8))
    a = b.copy()
    a[1, 2, 4] *= 1.5
    e = grading.row_rel_l2(a, b).reshape(2, 3, 5)
    assert e[1, 2, 4] == pytest.approx(0.5)
    assert np.count_nonzero(e) == 1


def test_a_wrong_row_hides_in_the_global_error_but_not_in_the_row_bound():
    rng = np.random.default_rng(2)
    b = rng.standard_normal((10000, 128))
    a = b.copy()
    a[4321] *= 1.5                       # one row carries 50 % too much mass
    assert grading.rel_l2(a, b) < 1e-2   # passes the global bf16 bound ...
    assert grading.max_row_rel_l2(a, b) > grading.ROW_FACTOR * 1e-2   # ... not the row bound
