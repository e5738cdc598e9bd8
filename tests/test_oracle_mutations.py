"""Planted mistakes in the oracle must fail at least one pin.

Each case copies the oracle's source, applies one plausible slip (a flipped
comparison, a dropped rescale, a wrong head or causal index, ...), loads the
mutant on the CPU and runs a battery of the pin tests against it.  A mutant
that passes every pin would mean the pins cannot tell it from the real
oracle.
"""

import types

import pytest

import oracle
import oracle.attention as attention
from tests import test_oracle_pins as pins  # noqa: E402

EXPORTS = ["decode", "dense_decode", "dense_prefill", "log_threshold", "lse_combine", "n_tiles",
           "prefill", "skip_fraction", "split_ranges", "stream_pass", "to_f64", "visit_order"]

MUTATIONS = {
    "non-strict comparison": ("skip = np.full(rows, delta < ln_thr)",
                              "skip = np.full(rows, delta <= ln_thr)"),
    "skipped tile leaves m alone": ("            m = m_new\n",
                                    "            m = np.where(keep, m_new, m)\n"),
    "top-left causal alignment": ("rows[:, None] + (Lk - Lq)] = NEG_INF",
                                  "rows[:, None]] = NEG_INF"),
    "kv head h % Hkv": ("hk = h // g\n", "hk = h % Hkv\n"),
    "no rescale of l": ("l = alpha * l + ", "l = l + "),
    "no rescale of O": ("O = alpha[:, None] * O + ", "O = O + "),
    "skipped tile still adds to l": ("np.where(keep, p.sum(axis=1), 0.0)", "p.sum(axis=1)"),
    "delta sign flipped": ("tile_max - m))", "m - tile_max))"),
    "uniform takes min over rows": ("delta = float(delta_r.max())", "delta = float(delta_r.min())"),
    "first visible tile may be skipped": ("np.where(m == NEG_INF, math.inf, tile_max - m)",
                                          "np.where(m == NEG_INF, NEG_INF, tile_max - m)"),
    "floor split size": ("per = -(-nK // S)", "per = max(1, nK // S)"),
    "lse combine ignores weights": ("wn = np.where(fin[None, :], w / np.where(fin, tot, 1.0)[None, :], 0.0)",
                                    "wn = np.full_like(w, 1.0 / w.shape[0])"),
    "diag_first causal ascending": ("            return tiles[::-1]", "            return tiles"),
    "wrong tile of a key": ("keys = np.arange(j * tk, min((j + 1) * tk, Lk))",
                            "keys = np.arange(j * tk, min((j + 1) * tk + 1, Lk))"),
    "natural-log threshold replaced by log10": ("math.log(thr)", "math.log10(thr)"),
    "natural-log threshold replaced by log2": ("math.log(thr)", "math.log2(thr)"),
}


def mutant(old, new):
    with open(attention.__file__) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def battery():
    yield lambda: [pins.test_hand_worked_example(c) for c in range(10)]
    yield pins.test_ties_are_kept
    yield lambda: pins.test_threshold_zero_is_softmax_attention_prefill(True, "ascending",
                                                                        (200, 333, 128, 128))
    yield lambda: pins.test_threshold_zero_is_softmax_attention_prefill(False, "diag_first",
                                                                        (333, 200, 64, 32))
    yield lambda: pins.test_threshold_zero_is_softmax_attention_decode(3, False)
    yield lambda: pins.test_threshold_at_least_one_keeps_only_record_tiles(1.0, "diag_first", True)
    yield lambda: pins.test_threshold_at_least_one_keeps_only_record_tiles(2.5, "ascending", False)
    yield lambda: [pins.test_brute_force_mask_enumeration(s, t, 4) for s in range(3)
                   for t in (0.05, 1.0, 3.0)]
    yield lambda: pins.test_brute_force_per_row_and_splits(0, 0.5)
    yield pins.test_visit_orders
    yield pins.test_split_ranges
    yield pins.test_uniform_skips_only_where_every_row_skips
    yield lambda: pins.test_gumbel_scores_skip_fraction_matches_closed_form(4096, 64.0, 128)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    mod = mutant(*MUTATIONS[name])
    for e in EXPORTS:
        monkeypatch.setattr(oracle, e, getattr(mod, e))
    caught = []
    for check in battery():
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"no pin caught the planted mistake: {name}"


def test_unmutated_battery_passes():
    for check in battery():
        check()


# --------------------------------------------------------------------------- backward

from tests import test_oracle_backward_pins as bpins  # noqa: E402

BACKWARD_MUTATIONS = {
    "softmax derivative without the row term": ("ds = p * (dp - d[:, None])", "ds = p * dp"),
    "key gradient without the scale": ("dk[b, hk] += scale * (ds.T @ q[b, h, rows])",
                                       "dk[b, hk] += ds.T @ q[b, h, rows]"),
    "value gradient from dS": ("dv[b, hk] += p.T @ dor", "dv[b, hk] += ds.T @ dor"),
    "skipped tiles kept": ("if m is None or m[b, h, i, j] == MASK_COMPUTED:",
                           "if m is None or m[b, h, i, j] != MASK_UNVISITED:"),
    "top-left causal alignment": ("keys_all[None, :] <= rows[:, None] + (Lk - Lq)",
                                  "keys_all[None, :] <= rows[:, None]"),
    "query gradient from P instead of dS": ("dq[b, h, rows] = scale * (ds @ k[b, hk])",
                                            "dq[b, h, rows] = scale * (p @ k[b, hk])"),
}


def backward_battery():
    yield lambda: bpins.test_dense_gradients_match_autograd(True, dict(Lq=130, Lk=300))
    yield lambda: bpins.test_dense_gradients_match_autograd(False, dict(Hq=4, Hkv=2, Lq=200,
                                                                        Lk=200))
    yield lambda: bpins.test_skip_gradients_match_finite_differences_of_the_forward(1.0, True)
    yield bpins.test_key_gradient_sums_to_zero
    yield bpins.test_value_gradient_sums_to_the_output_gradient


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_planted_mistake(name, monkeypatch):
    mod = mutant(*BACKWARD_MUTATIONS[name])
    monkeypatch.setattr(oracle, "prefill_backward", mod.prefill_backward)
    caught = []
    for check in backward_battery():
        try:
            check()
        except AssertionError:
            caught.append(check)
    assert caught, f"no backward pin caught the planted mistake: {name}"


def test_unmutated_backward_battery_passes():
    for check in backward_battery():
        check()


# --------------------------------------------------------------------------- grader

import oracle.grading as grading  # noqa: E402
from tests import test_grading_pins as gpins  # noqa: E402

GRADING_MUTATIONS = {
    "far-flip term dropped": ('"ok": bool(far_diff.sum() == 0 and agree >= MIN_AGREEMENT)',
                              '"ok": bool(agree >= MIN_AGREEMENT)'),
    "agreement bound dropped": ('"ok": bool(far_diff.sum() == 0 and agree >= MIN_AGREEMENT)',
                                '"ok": bool(far_diff.sum() == 0)'),
    "statistic read in log2 units": ("r = np.exp(d) / thr", "r = np.exp2(d) / thr"),
    "margin inverted": ("near = np.abs(r - 1.0) <= NEAR_REL", "near = np.abs(r - 1.0) > NEAR_REL"),
    "absolute instead of relative margin": ("near = np.abs(r - 1.0) <= NEAR_REL",
                                            "near = np.abs(np.exp(d) - thr) <= NEAR_REL"),
    "selection ignored": ("diff = (g != r) & sel", "diff = (g != r)"),
    "zero threshold makes every tile near": ("    if thr <= 0:\n        return np.zeros(d.shape, bool)\n",
                                             "    if thr <= 0:\n        return np.ones(d.shape, bool)\n"),
    "relative error against the wrong operand": (
        "return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))",
        "return float(np.linalg.norm(a - b) / max(np.linalg.norm(a), 1e-300))"),
    "row bound takes the mean": ("return float(e.max()) if e.size else 0.0",
                                 "return float(e.mean()) if e.size else 0.0"),
    "row errors over columns": ("return np.linalg.norm(a2 - b2, axis=1) / np.maximum(nb, floor)",
                                "return np.linalg.norm(a2 - b2) / np.maximum(nb, floor)"),
}


def grading_mutant(old, new):
    with open(grading.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("grading_mutant")
    exec(compile(src.replace(old, new), "grading_mutant", "exec"), mod.__dict__)
    return mod


def grading_battery():
    for name in dir(gpins):
        fn = getattr(gpins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        if name == "test_near_band_is_relative_one_in_a_thousand_in_natural_log_units":
            for thr in (1e-4, 0.01, 0.7105, 1.0, 3.0):
                yield lambda fn=fn, thr=thr: fn(thr)
        elif name == "test_near_flips_above_one_in_a_thousand_fail":
            for flips, ok in ((10, True), (11, False), (20, False)):
                yield lambda fn=fn, flips=flips, ok=ok: fn(flips, ok)
        else:
            yield fn


@pytest.mark.parametrize("name", sorted(GRADING_MUTATIONS))
def test_grading_pins_catch_planted_mistake(name, monkeypatch):
    mod = grading_mutant(*GRADING_MUTATIONS[name])
    for e in ("near_threshold", "grade_masks", "rel_l2", "row_rel_l2", "max_row_rel_l2"):
        monkeypatch.setattr(grading, e, getattr(mod, e))
    caught = []
    for check in grading_battery():
        try:
            check()
        except (AssertionError, ValueError):
            caught.append(check)
    assert caught, f"no grader pin caught the planted mistake: {name}"


def test_unmutated_grading_battery_passes():
    n = 0
    for check in grading_battery():
        check()
        n += 1
    assert n >= 15
