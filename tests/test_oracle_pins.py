"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

None of these tests re-derives the oracle's streaming pass: each compares it
with something else -- a library softmax (scipy), a hand-worked example, an
exp-free scan over tile maxima, brute-force enumeration of skip masks from the
rule's definition, or an inequality the rule implies.

Page references: the vLLM-Omni design page "Skip-Softmax" and the BLASST
summary page (arXiv 2512.12087).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from synth import clustered_decode, clustered_prefill, gumbel_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers

def softmax_attention(qr, kr, vr, scale, visible):
    """Textbook attention through scipy's softmax; rows that see no key give 0."""
    s = scale * (qr @ kr.T)
    out = np.zeros((qr.shape[0], vr.shape[1]))
    for r in range(qr.shape[0]):
        if visible[r].any():
            w = softmax(np.where(visible[r], s[r], -np.inf))
            out[r] = w @ vr
    return out


def causal_visible(Lq, Lk, causal):
    rows = np.arange(Lq)[:, None]
    keys = np.arange(Lk)[None, :]
    if causal:
        return keys <= rows + (Lk - Lq)
    return np.ones((Lq, Lk), bool)


def prefill_inputs(seed, B=1, Hq=2, Hkv=1, Lq=300, Lk=300, D=16, Dv=8, r=4.0, n_c=6,
                   mode="tile"):
    x = clustered_prefill(seed, B, Hq, Hkv, Lq, Lk, D, Dv, n_c, r, query_mode=mode,
                          dtype="f32")
    return oracle.to_f64(x["q"]), oracle.to_f64(x["k"]), oracle.to_f64(x["v"])


def rel_err(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------- hand example

def _hand():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", range(len(_hand()["cases"])))
def test_hand_worked_example(case):
    """Masks and outputs worked by hand from the skip rule (design page, 'The skip
    test'; BLASST summary, 'Kerninzicht'), including the split restart of the
    running max and the thr > 1 case where a skipped tile raises m."""
    h = _hand()
    c = h["cases"][case]
    q = np.array(h["q"]).reshape(1, 1, 1)
    k = np.array(h["k"]).reshape(1, 1, -1, 1)
    v = np.array(h["v"]).reshape(1, 1, -1, 1)
    res = oracle.decode(q, k, v, 1.0, c["threshold"], c["splits"], tk=h["tile"])
    assert res["mask"][0, 0].tolist() == c["mask"]
    kept = c["kept_keys"]
    s = np.array(h["k"])[kept]
    want = sum(math.exp(si) * (kk + 1) for si, kk in zip(s, kept)) / sum(math.exp(si) for si in s)
    assert abs(res["out"][0, 0, 0] - want) < 1e-13 * abs(want)
    if c["splits"] == 1:  # the same row through the prefill entry
        p = oracle.prefill(q.reshape(1, 1, 1, 1), k, v, 1.0, False, c["threshold"], tq=1,
                           tk=h["tile"])
        assert p["mask"][0, 0, 0].tolist() == c["mask"]
        assert abs(p["out"][0, 0, 0, 0] - want) < 1e-13 * abs(want)


# --------------------------------------------------------------------------- threshold 0

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["ascending", "diag_first"])
@pytest.mark.parametrize("shape", [(300, 300, 128, 128), (200, 333, 128, 128),
                                   (333, 200, 64, 32), (97, 250, 32, 64)])
def test_threshold_zero_is_softmax_attention_prefill(causal, order, shape):
    """At threshold 0 nothing is skipped and the single pass with rescaling is
    exact (design page, 'The online-softmax pass'): it must equal textbook
    softmax attention, bottom-right causal, with GQA head sharing."""
    Lq, Lk, tq, tk = shape
    q, k, v = prefill_inputs(11, B=2, Hq=4, Hkv=2, Lq=Lq, Lk=Lk)
    res = oracle.prefill(q, k, v, 0.3, causal, 0.0, tq=tq, tk=tk, order=order)
    vis = causal_visible(Lq, Lk, causal)
    for b in range(2):
        for h in range(4):
            ref = softmax_attention(q[b, h], k[b, h // 2], v[b, h // 2], 0.3, vis)
            assert rel_err(res["out"][b, h], ref) < 1e-12
    assert not (res["mask"] == oracle.MASK_SKIPPED).any()


@pytest.mark.parametrize("mode", ["uniform", "per_row"])
def test_threshold_zero_per_row_and_no_visible_rows(mode):
    """Rows that see no key (causal, Lq > Lk) give 0; per_row mode at 0 is exact too."""
    q, k, v = prefill_inputs(12, Hq=2, Hkv=2, Lq=300, Lk=100)
    res = oracle.prefill(q, k, v, 0.25, True, 0.0, tq=64, tk=32, mode=mode)
    vis = causal_visible(300, 100, True)
    assert not vis[:200].any()
    for h in range(2):
        ref = softmax_attention(q[0, h], k[0, h], v[0, h], 0.25, vis)
        assert rel_err(res["out"][0, h], ref) < 1e-12
        assert np.all(res["out"][0, h, :200] == 0)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 100])
@pytest.mark.parametrize("latent", [False, True])
def test_threshold_zero_is_softmax_attention_decode(splits, latent):
    """Split-KV decode at threshold 0: every split is exact and the log-sum-exp
    merge reproduces the full softmax over all keys."""
    x = clustered_decode(21, 2, 8, 2, 1000, 24, 16, 8, 3.0, latent=latent, dtype="f32")
    q, k = oracle.to_f64(x["q"]), oracle.to_f64(x["k"])
    v = None if latent else oracle.to_f64(x["v"])
    res = oracle.decode(q, k, v, 0.2, 0.0, splits, latent_dv=16 if latent else None)
    vv = k[..., :16] if latent else v
    for b in range(2):
        for h in range(8):
            ref = softmax_attention(q[b, h][None], k[b, h // 4], vv[b, h // 4], 0.2,
                                    np.ones((1, 1000), bool))[0]
            assert rel_err(res["out"][b, h], ref) < 1e-12
    per = -(-8 // min(splits, 8))
    assert res["splits"] == [(t, min(t + per, 8)) for t in range(0, 8, per)]


# --------------------------------------------------------------------------- threshold >= 1

def tile_max_records(tile_max, seen, margin):
    """Exp-free scan: a tile survives iff some row that sees a key in it has
    tile_max - (max of that row's earlier tile maxima) >= margin."""
    R, T = tile_max.shape
    best = np.full(R, -np.inf)
    keep = []
    for t in range(T):
        kk = False
        for r in range(R):
            if seen[r, t] and (best[r] == -np.inf or tile_max[r, t] - best[r] >= margin):
                kk = True
        keep.append(kk)
        best = np.maximum(best, tile_max[:, t])
    return keep


@pytest.mark.parametrize("thr", [1.0, 2.5])
@pytest.mark.parametrize("order", ["ascending", "diag_first"])
@pytest.mark.parametrize("causal", [False, True])
def test_threshold_at_least_one_keeps_only_record_tiles(thr, order, causal):
    """At threshold >= 1 a tile survives only if it raises some row's running max
    by at least ln(threshold): the test exp(tile_max - running_max) < threshold
    (design page, 'The skip test') written as a scan over tile maxima.  The
    output is softmax attention over the surviving tiles' keys."""
    Lq, Lk, tq, tk = 200, 333, 64, 32
    q, k, v = prefill_inputs(31, Hq=2, Hkv=1, Lq=Lq, Lk=Lk, r=2.0)
    res = oracle.prefill(q, k, v, 0.3, causal, thr, tq=tq, tk=tk, order=order)
    vis = causal_visible(Lq, Lk, causal)
    nQ, nK = oracle.n_tiles(Lq, tq), oracle.n_tiles(Lk, tk)
    for h in range(2):
        s = 0.3 * q[0, h] @ k[0, 0].T
        s = np.where(vis, s, -np.inf)
        for i in range(nQ):
            rows = slice(i * tq, min((i + 1) * tq, Lq))
            tiles = oracle.visit_order(i, nK, Lq, Lk, causal, order, tq, tk)
            tm = np.stack([s[rows, j * tk:(j + 1) * tk].max(axis=1) for j in tiles], axis=1)
            seen = np.stack([vis[rows, j * tk:(j + 1) * tk].any(axis=1) for j in tiles], axis=1)
            keep = tile_max_records(tm, seen, math.log(thr))
            got = [res["mask"][0, h, i, j] == 0 for j in tiles]
            assert got == keep
            kept_vis = np.zeros_like(vis[rows])
            for j, kk in zip(tiles, keep):
                if kk:
                    kept_vis[:, j * tk:(j + 1) * tk] = vis[rows, j * tk:(j + 1) * tk]
            ref = softmax_attention(q[0, h][rows], k[0, 0], v[0, 0], 0.3, kept_vis)
            assert rel_err(res["out"][0, h][rows], ref) < 1e-12


# --------------------------------------------------------------------------- soundness

def dense_weights(qr, kr, scale, visible):
    s = np.where(visible, scale * (qr @ kr.T), -np.inf)
    w = np.zeros_like(s)
    for r in range(s.shape[0]):
        if visible[r].any():
            w[r] = softmax(s[r])
    return w


@pytest.mark.parametrize("thr", [1e-4, 1e-2, 0.2, 0.9])
@pytest.mark.parametrize("mode", ["uniform", "per_row"])
@pytest.mark.parametrize("order", ["ascending", "diag_first"])
def test_skipped_keys_have_dense_weight_below_threshold_prefill(thr, mode, order):
    """exp(tile_max - running_max) bounds the softmax weight of every key in the
    tile (design page, 'The skip test'): each skipped key's weight under dense
    softmax is < threshold."""
    Lq, Lk, tq, tk = 256, 512, 64, 32
    q, k, v = prefill_inputs(44, Hq=2, Hkv=1, Lq=Lq, Lk=Lk, r=8.0)
    nskip = 0
    for causal in (True, False):
        res = oracle.prefill(q, k, v, 0.35, causal, thr, tq=tq, tk=tk, mode=mode, order=order)
        vis = causal_visible(Lq, Lk, causal)
        for h in range(2):
            w = dense_weights(q[0, h], k[0, 0], 0.35, vis)
            for r in range(Lq):
                i = r // tq
                for j in range(oracle.n_tiles(Lk, tk)):
                    code = (res["mask"][0, h, i, j] if mode == "uniform"
                            else res["row_mask"][0, h, r, j])
                    if code == oracle.MASK_SKIPPED:
                        nskip += 1
                        assert w[r, j * tk:(j + 1) * tk].max() < thr
    assert nskip > 0


@pytest.mark.parametrize("thr", [1e-3, 0.05, 0.5])
@pytest.mark.parametrize("splits", [1, 3])
def test_skipped_keys_have_dense_weight_below_threshold_decode(thr, splits):
    x = clustered_decode(51, 2, 8, 2, 2000, 32, 16, 16, 7.0, dtype="f32")
    q, k, v = (oracle.to_f64(x[n]) for n in "qkv")
    res = oracle.decode(q, k, v, 0.18, thr, splits, tk=64)
    nskip = 0
    for b in range(2):
        for h in range(8):
            w = dense_weights(q[b, h][None], k[b, h // 4], 0.18, np.ones((1, 2000), bool))[0]
            for j in range(oracle.n_tiles(2000, 64)):
                if res["mask"][b, h // 4, j] == oracle.MASK_SKIPPED:
                    nskip += 1
                    assert w[j * 64:(j + 1) * 64].max() < thr
    assert nskip > 0


# --------------------------------------------------------------------------- brute force

def brute_force_masks(s_tiles, thr, reading, per_row_row=None):
    """All masks over the visited tiles that are self-consistent under the skip
    rule evaluated from its definition: tile t is skipped iff, for every row
    that sees a key in it, exp(tile_max - m) < thr, with m recomputed from
    scratch as the max of every score of the tiles visited before t
    (reading "all") or of the tiles that the mask keeps (reading "kept").
    A row that has seen no score yet (m = -inf) always keeps the tile."""
    T = len(s_tiles)
    rows = range(s_tiles[0].shape[0]) if per_row_row is None else [per_row_row]
    found = []
    for bits in itertools.product([0, 1], repeat=T):
        ok = True
        for t in range(T):
            prev = [u for u in range(t) if reading == "all" or bits[u] == 0]
            rule_skip = True
            for r in rows:
                tm = s_tiles[t][r].max()
                if tm == -np.inf:
                    if thr == 0:  # exp(-inf) = 0 is not < 0
                        rule_skip = False
                    continue
                m = max([s_tiles[u][r].max() for u in prev], default=-np.inf)
                if m == -np.inf or not (math.exp(tm - m) < thr):
                    rule_skip = False
            if rule_skip != bool(bits[t]):
                ok = False
                break
        if ok:
            found.append(list(bits))
    return found


def _tiny_tiles(seed, R, nT, tk, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((nT * tk, D)) * rng.uniform(0.2, 2.5, size=(nT * tk, 1))
    return q, k


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("thr", [0.0, 0.05, 0.3, 1.0, 3.0])
@pytest.mark.parametrize("tk", [4, 8])
def test_brute_force_mask_enumeration(seed, thr, tk):
    """Exactly one mask is consistent with the rule; it is the oracle's.  For
    threshold <= 1 the 'kept tiles only' reading of the running max gives the
    same mask; for threshold > 1 only the 'every visited tile' reading must."""
    nT = 11 if tk == 4 else 9
    R, D = 3, 6
    q, k = _tiny_tiles(1000 * seed + tk, R, nT, tk, D)
    v = np.random.default_rng(seed).standard_normal((nT * tk, 5))
    res = oracle.prefill(q[None, None], k[None, None], v[None, None], 0.9, False, thr,
                         tq=R, tk=tk)
    mask = [int(x) for x in res["mask"][0, 0, 0]]
    s_tiles = [0.9 * q @ k[j * tk:(j + 1) * tk].T for j in range(nT)]
    a = brute_force_masks(s_tiles, thr, "all")
    assert a == [mask]
    b = brute_force_masks(s_tiles, thr, "kept")
    assert len(b) == 1
    if thr <= 1:
        assert b == [mask]
    keep_keys = np.concatenate([np.arange(j * tk, (j + 1) * tk) for j in range(nT) if mask[j] == 0])
    vis = np.zeros((R, nT * tk), bool)
    vis[:, keep_keys] = True
    ref = softmax_attention(q, k, v, 0.9, vis)
    assert rel_err(res["out"][0, 0, 0:R], ref) < 1e-12


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("thr", [0.05, 0.5])
def test_brute_force_per_row_and_splits(seed, thr):
    """Per-row decisions and split-KV decode, each against enumeration: every row
    alone (per_row) and every split alone (decode) has exactly one consistent
    mask, and it is the oracle's."""
    tk, nT, R, D = 4, 10, 3, 5
    q, k = _tiny_tiles(77 + seed, R, nT, tk, D)
    v = np.random.default_rng(seed).standard_normal((nT * tk, 4))
    s_tiles = [0.8 * q @ k[j * tk:(j + 1) * tk].T for j in range(nT)]
    res = oracle.prefill(q[None, None], k[None, None], v[None, None], 0.8, False, thr, tq=R,
                         tk=tk, mode="per_row")
    for r in range(R):
        assert brute_force_masks(s_tiles, thr, "all", per_row_row=r) == [
            [int(x) for x in res["row_mask"][0, 0, r]]]
    for S in (2, 3):
        dec = oracle.decode(q[None], k[None, None], v[None, None], 0.8, thr, S, tk=tk)
        for t0, t1 in oracle.split_ranges(nT, S):
            want = brute_force_masks(s_tiles[t0:t1], thr, "all")
            assert want == [[int(x) for x in dec["mask"][0, 0, t0:t1]]]


# --------------------------------------------------------------------------- invariants

def test_skip_is_monotone_in_threshold():
    """Skip sets grow with the threshold on [0, 1] (the test is exp(.) < thr)."""
    q, k, v = prefill_inputs(61, Hq=2, Hkv=1, Lq=400, Lk=400, r=6.0)
    prev = None
    for thr in [0.0, 1e-4, 1e-3, 1e-2, 0.05, 0.2, 0.5, 1.0]:
        m = oracle.prefill(q, k, v, 0.3, True, thr, tq=64, tk=32)["mask"] == 1
        if prev is not None:
            assert np.all(m >= prev)
        prev = m


def gumbel_expected_skip(L, a, tk=128):
    """Expected skip fraction of one streaming pass over ``L`` keys whose
    scaled scores are i.i.d. standard Gumbel, at threshold ``a / L``.

    The maximum of n i.i.d. Gumbel(0, 1) draws is ln n + Gumbel(0, 1) (the
    family is max-stable), so before tile j+1 (j full tiles seen) the running
    max is ln(tk j) + G1 and the tile max is ln(tk) + G2, with G1 and G2
    independent.  G1 - G2 is logistic, and exp(tile max - running max) < a / L
    holds with probability a j / (a j + L).  Tile 1 is never skipped.  The
    sum over tiles depends on L only through the tile count, so for a fixed
    ``a`` the skip fraction is (up to a 1/n term) the same at every length:
    the threshold scaling 1/L keeps sparsity stable exactly when scores have
    this unit exponential tail.
    """
    n = L // tk
    j = np.arange(1, n)
    return float((a * j / (a * j + L)).sum() / n)


@pytest.mark.parametrize("L,a,streams", [(4096, 3000.0, 96), (8192, 900.0, 96),
                                         (4096, 64.0, 128)])
def test_gumbel_scores_skip_fraction_matches_closed_form(L, a, streams):
    """Sample mean of the per-stream skip fraction within 4 standard errors
    of the closed form (threshold a/L scaled by the sequence length, the
    BLASST summary page, "Calibratie en Thresholding")."""
    D = 64
    B, Hkv = streams // 4, 4
    x = gumbel_decode(81 + L, B, Hkv, Hkv, L, D, 16, 1 / math.sqrt(D), dtype="f32")
    q, k, v = (oracle.to_f64(x[n]) for n in "qkv")
    mask = oracle.decode(q, k, v, 1 / math.sqrt(D), a / L, 1)["mask"]
    per_stream = (mask == 1).mean(axis=2).ravel()
    se = per_stream.std(ddof=1) / math.sqrt(per_stream.size)
    want = gumbel_expected_skip(L, a)
    assert abs(per_stream.mean() - want) <= 4 * se, (per_stream.mean(), want, se)


def test_split_refinement_only_shrinks_skip_set():
    """Each split restarts its running max, and a split's prefix max is <= the
    full prefix max, so refining the split partition can only un-skip tiles."""
    x = clustered_decode(71, 2, 8, 2, 4096, 32, 16, 16, 7.0, dtype="f32")
    q, k, v = (oracle.to_f64(x[n]) for n in "qkv")
    for thr in [1e-3, 0.05, 0.5]:
        s1 = oracle.decode(q, k, v, 0.18, thr, 1, tk=64)["mask"] == 1
        s4 = oracle.decode(q, k, v, 0.18, thr, 4, tk=64)["mask"] == 1   # 16 tiles each
        s16 = oracle.decode(q, k, v, 0.18, thr, 16, tk=64)["mask"] == 1  # refines 4
        assert np.all(s4 <= s1) and np.all(s16 <= s4)
        assert s1.sum() > 0


@pytest.mark.parametrize("thr", [1e-3, 3e-2, 0.3])
def test_output_error_bounded_by_dropped_mass(thr):
    """Per row, ||O_dense - O_skip|| <= 2 * eps * max||v|| where eps is the dense
    softmax mass of the skipped keys, and eps < (#skipped keys) * threshold."""
    Lq, Lk, tq, tk = 256, 512, 64, 32
    q, k, v = prefill_inputs(81, Hq=1, Hkv=1, Lq=Lq, Lk=Lk, r=5.0)
    res = oracle.prefill(q, k, v, 0.3, False, thr, tq=tq, tk=tk)
    vis = np.ones((Lq, Lk), bool)
    w = dense_weights(q[0, 0], k[0, 0], 0.3, vis)
    dense = softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.3, vis)
    vmax = np.linalg.norm(v[0, 0], axis=1).max()
    for r in range(Lq):
        sk = [j for j in range(Lk // tk) if res["mask"][0, 0, r // tq, j] == 1]
        keys = np.concatenate([np.arange(j * tk, (j + 1) * tk) for j in sk]) if sk else []
        eps = w[r, keys].sum() if len(keys) else 0.0
        assert eps <= len(keys) * thr
        assert np.linalg.norm(dense[r] - res["out"][0, 0, r]) <= 2 * eps * vmax + 1e-12


# --------------------------------------------------------------------------- special cases

def test_gqa_equals_mha_with_repeated_kv():
    """Query head h reads KV head h // g: GQA equals MHA with KV repeated per head."""
    q, k, v = prefill_inputs(91, Hq=6, Hkv=2, Lq=260, Lk=260, r=6.0)
    krep, vrep = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    for thr in [0.0, 0.02]:
        a = oracle.prefill(q, k, v, 0.3, True, thr, tq=64, tk=32)
        b = oracle.prefill(q, krep, vrep, 0.3, True, thr, tq=64, tk=32)
        assert np.array_equal(a["mask"], b["mask"])
        assert np.array_equal(a["out"], b["out"])


def test_mqa_decode_equals_per_head_decodes():
    """MQA (one KV head) in per_row mode equals separate single-head decodes."""
    x = clustered_decode(92, 1, 4, 1, 900, 16, 8, 8, 6.0, dtype="f32")
    q, k, v = (oracle.to_f64(x[n]) for n in "qkv")
    full = oracle.decode(q, k, v, 0.25, 0.05, 2, tk=64, mode="per_row")
    for h in range(4):
        one = oracle.decode(q[:, h:h + 1], k, v, 0.25, 0.05, 2, tk=64)
        assert np.array_equal(one["mask"][0, 0], full["row_mask"][0, h])
        assert np.allclose(one["out"][0, 0], full["out"][0, h], rtol=0, atol=1e-15)


def test_decode_one_split_equals_prefill_row_block():
    """Decode with one split is the prefill pass over one row block made of the
    group's query heads."""
    x = clustered_decode(93, 2, 8, 2, 1100, 16, 8, 8, 6.0, dtype="f32")
    q, k, v = (oracle.to_f64(x[n]) for n in "qkv")
    for thr in [0.0, 0.01, 0.3]:
        d = oracle.decode(q, k, v, 0.25, thr, 1, tk=128)
        for b in range(2):
            for hk in range(2):
                p = oracle.prefill(q[b, hk * 4:(hk + 1) * 4][None, None], k[b, hk][None, None],
                                   v[b, hk][None, None], 0.25, False, thr, tq=4, tk=128)
                assert np.array_equal(p["mask"][0, 0, 0], d["mask"][b, hk])
                assert np.allclose(p["out"][0, 0], d["out"][b, hk * 4:(hk + 1) * 4], atol=1e-14)


def test_per_row_with_one_row_block_equals_uniform():
    q, k, v = prefill_inputs(94, Hq=1, Hkv=1, Lq=64, Lk=640, r=6.0)
    for thr in [0.01, 0.2]:
        u = oracle.prefill(q, k, v, 0.3, False, thr, tq=1, tk=32)
        p = oracle.prefill(q, k, v, 0.3, False, thr, tq=1, tk=32, mode="per_row")
        assert np.array_equal(u["mask"][0, 0], p["row_mask"][0, 0])
        assert np.array_equal(u["out"], p["out"])


def test_uniform_skips_only_where_every_row_skips():
    """Uniform granularity: a tile is skipped for the block iff every row of the
    block would skip it on its own (same running maxima, since m is updated on
    skipped tiles too)."""
    q, k, v = prefill_inputs(95, Hq=2, Hkv=1, Lq=256, Lk=512, r=6.0)
    for thr in [0.01, 0.3]:
        u = oracle.prefill(q, k, v, 0.3, True, thr, tq=64, tk=32)
        p = oracle.prefill(q, k, v, 0.3, True, thr, tq=64, tk=32, mode="per_row")
        rm = p["row_mask"]
        for i in range(4):
            blk = rm[0, :, i * 64:(i + 1) * 64, :]
            allskip = (blk == 1).all(axis=1)
            assert np.array_equal(u["mask"][0, :, i, :] == 1, allskip)


def test_force_mask_replays_decisions():
    """Forcing the oracle's own mask reproduces its output; forcing all-computed
    reproduces dense attention."""
    q, k, v = prefill_inputs(96, Hq=2, Hkv=1, Lq=200, Lk=300, r=6.0)
    a = oracle.prefill(q, k, v, 0.3, True, 0.05, tq=64, tk=32)
    b = oracle.prefill(q, k, v, 0.3, True, 0.05, tq=64, tk=32, force_mask=a["mask"])
    assert np.array_equal(a["out"], b["out"])
    z = np.where(a["mask"] == 1, 0, a["mask"])
    c = oracle.prefill(q, k, v, 0.3, True, 0.05, tq=64, tk=32, force_mask=z)
    assert rel_err(c["out"], oracle.dense_prefill(q, k, v, 0.3, True)) < 1e-12


def test_dense_references_match_library_softmax():
    q, k, v = prefill_inputs(97, Hq=2, Hkv=1, Lq=150, Lk=120)
    d = oracle.dense_prefill(q, k, v, 0.3, True)
    vis = causal_visible(150, 120, True)
    for h in range(2):
        assert rel_err(d[0, h], softmax_attention(q[0, h], k[0, 0], v[0, 0], 0.3, vis)) < 1e-12
    x = clustered_decode(98, 1, 4, 2, 300, 16, 16, 4, 3.0, latent=True, dtype="f32")
    qq, kk = oracle.to_f64(x["q"]), oracle.to_f64(x["k"])
    dd = oracle.dense_decode(qq, kk, None, 0.25, latent_dv=8)
    for h in range(4):
        ref = softmax_attention(qq[0, h][None], kk[0, h // 2], kk[0, h // 2, :, :8], 0.25,
                                np.ones((1, 300), bool))[0]
        assert rel_err(dd[0, h], ref) < 1e-12


def test_visit_orders():
    """diag_first: causal goes from the block's last visible tile down to 0;
    non-causal starts at the block's own tile and wraps."""
    assert oracle.visit_order(3, 8, 1024, 1024, True, "ascending", 128, 128) == [0, 1, 2, 3]
    assert oracle.visit_order(3, 8, 1024, 1024, True, "diag_first", 128, 128) == [3, 2, 1, 0]
    assert oracle.visit_order(5, 8, 1024, 1024, False, "diag_first", 128, 128) == [5, 6, 7, 0, 1, 2, 3, 4]
    # bottom-right alignment: 100 queries against 300 keys, last row sees key 299
    assert oracle.visit_order(0, 3, 100, 300, True, "ascending", 128, 128) == [0, 1, 2]
    # 300 queries against 100 keys: the first 200 rows see nothing
    assert oracle.visit_order(0, 1, 300, 100, True, "ascending", 128, 128) == []
    assert oracle.visit_order(1, 1, 300, 100, True, "ascending", 128, 128) == [0]


def test_split_ranges():
    assert oracle.split_ranges(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert oracle.split_ranges(9, 4) == [(0, 3), (3, 6), (6, 9)]
    assert oracle.split_ranges(5, 99) == [(i, i + 1) for i in range(5)]
    assert oracle.split_ranges(256, 8) == [(32 * i, 32 * i + 32) for i in range(8)]


# --------------------------------------------------------------------------- host formulas

def test_host_formulas():
    """Design page, 'The threshold': threshold = factor / seqlen; calibrated
    factor a*exp(b*s); direct factor = threshold * seqlen."""
    assert oracle.factor_calibrated(2.0, 0.0, 0.7) == 2.0
    assert abs(oracle.factor_calibrated(1.5, math.log(2.0), 1.0) - 3.0) < 1e-15
    assert abs(oracle.factor_calibrated(1.0, 2.0, 0.5) - math.e) < 1e-15
    assert oracle.factor_direct(1e-3, 32768) == pytest.approx(32.768, rel=1e-15)
    assert oracle.threshold(32.768, 32768) == pytest.approx(1e-3, rel=1e-15)
    assert oracle.threshold(oracle.factor_direct(0.25, 4096), 4096) == 0.25


def test_gating_truth_table():
    """Design page, 'Timestep gating': dense while t > D, sparse once t <= D;
    a pipeline that publishes no timestep stays dense when D is set."""
    D = 0.7
    assert oracle.gate_enabled(1.0, D) is False
    assert oracle.gate_enabled(0.7, D) is True
    assert oracle.gate_enabled(0.6, D) is True
    assert oracle.gate_enabled(0.2, D) is True
    assert oracle.gate_enabled(None, D) is False
    assert oracle.gate_enabled(None, None) is True
    assert oracle.gate_enabled(0.95, None) is True


def test_ties_are_kept():
    """The comparison is strict (design page, 'The skip test': skip when the bound
    is *below* the threshold): at threshold 1 a tile whose max ties the running
    max is kept, one strictly below is skipped."""
    q = np.array([1.0]).reshape(1, 1, 1)
    k = np.array([0.0, -1.0, 0.0, -2.0, -1.0, -1.0]).reshape(1, 1, -1, 1)
    v = np.arange(1.0, 7.0).reshape(1, 1, -1, 1)
    res = oracle.decode(q, k, v, 1.0, 1.0, 1, tk=2)
    assert res["mask"][0, 0].tolist() == [0, 0, 1]
    s = np.array([0.0, -1.0, 0.0, -2.0])
    want = float(np.exp(s) @ np.arange(1.0, 5.0) / np.exp(s).sum())
    assert abs(res["out"][0, 0, 0] - want) < 1e-14
