"""fp64 CPU oracle for skip-softmax (BLASST) attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path.

What is computed, and where it comes from
-----------------------------------------
Sources: the vLLM-Omni design page "Skip-Softmax" (sections "The
online-softmax pass", "The skip test", "What this bounds", "The threshold",
"Timestep gating") and the summary page of arXiv 2512.12087 "BLASST: Dynamic
BLocked Attention Sparsity via Softmax Thresholding" (sections
"Kerninzicht", "Calibratie en Thresholding", "Kernel-ontwerp").

* One streaming pass over the keys in tiles of 128 keys.  Every query row
  keeps ``m`` (largest score seen so far), ``l`` (sum of exp(s - m)) and
  ``O`` (sum of exp(s - m) * v); ``l`` and ``O`` are rescaled by
  exp(m_old - m_new) whenever ``m`` grows, and the pass returns ``O / l``
  (design page, "The online-softmax pass").
* The tile scores ``S = Q K_j^T * scale`` are always computed, because the
  test needs the tile maximum (design page, "What this bounds").
* Skip test: a tile is skipped when exp(tile_max - running_max) < threshold,
  i.e. tile_max - running_max < ln(threshold) (design page, "The skip test";
  BLASST summary, "Kerninzicht", which states it as a log-domain comparison
  of the block maximum against the running maximum).  A skipped tile adds
  nothing to ``l`` or ``O``: no exponentials, no P.V, and in decode no V read.
* The decision is made per key tile; a single important key keeps the tile
  (design page, "What this bounds").

Readings where the pages leave a step open (each is also stated in the
design notes of the repository):

1. The test compares against the running max *before* the tile is folded in.
   For threshold <= 1 this gives the same decisions as the "after" reading.
2. A skipped tile still updates ``m`` (its scores were computed and ``m`` is
   the largest score seen so far).  For threshold <= 1 this never changes
   ``m``; for threshold > 1 (or a forced skip) ``l`` and ``O`` are rescaled
   so that the pass stays exact over the keys it kept.
3. The comparison is strict: threshold = 0 never skips.
4. Query-side granularity: ``mode="uniform"`` skips a tile only if every
   valid row of the row block passes (delta = max over rows of
   tile_max_r - m_r); ``mode="per_row"`` lets every row decide alone.  A
   prefill row block is a 128-row query tile of one head; a decode row block
   is the group of query heads that share one KV head.
5. Row statistic: delta_r = -inf when the row sees no key in the tile (it
   votes "skip"), +inf when the row has seen no key before (its first
   visible tile is never skipped), else tile_max_r - m_r.
6. Causal masking is bottom-right aligned: key c is visible to query row r
   iff c <= r + Lk - Lq.  Keys past Lk do not exist; rows past Lq do not
   vote.  Tiles with no visible key for any row of the block are not visited.
7. Visit order (not fixed by the pages): ``"ascending"`` key-tile order, or
   ``"diag_first"`` -- causal: the block's last visible tile first, then
   downwards to tile 0; non-causal: the block's own tile first, then upwards,
   wrapping to tile 0.
8. Split-KV decode: the key tiles are cut into contiguous splits of
   ceil(nK / S) tiles (the last may be shorter); every split is an
   independent streaming pass with its own running max, and the splits'
   (O_s / l_s, lse_s = m + ln l) are merged by the log-sum-exp combine.

Mask encoding: 0 = tile computed, 1 = tile skipped, 2 = tile not visited.
"""

from __future__ import annotations

import math

import numpy as np

MASK_COMPUTED = 0
MASK_SKIPPED = 1
MASK_UNVISITED = 2

NEG_INF = -math.inf


def to_f64(x):
    """Exact conversion of a bf16/fp32 torch tensor or a numpy array to fp64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def log_threshold(thr: float) -> float:
    """ln(threshold) with ln(0) = -inf, so a strict test at 0 never passes."""
    if not (thr >= 0.0):
        raise ValueError(f"threshold must be >= 0, got {thr!r}")
    return NEG_INF if thr == 0.0 else math.log(thr)


def n_tiles(L: int, T: int) -> int:
    return -(-L // T)


def split_ranges(nK: int, num_splits: int) -> list:
    """Contiguous splits of ceil(nK/S) tiles each; the last may be shorter.
    ``S`` is clamped to [1, nK]; empty trailing splits are dropped."""
    S = max(1, min(int(num_splits), nK))
    per = -(-nK // S)
    return [(s, min(s + per, nK)) for s in range(0, nK, per)]


def visit_order(i: int, nK: int, Lq: int, Lk: int, causal: bool, order: str,
                tq: int, tk: int) -> list:
    """Key tiles visited by query tile ``i``, in visit order (readings 6, 7)."""
    r0 = i * tq
    r1 = min((i + 1) * tq, Lq) - 1
    if causal:
        last_key = r1 + Lk - Lq
        if last_key < 0:
            return []
        tiles = list(range(0, min(nK - 1, last_key // tk) + 1))
        if order == "ascending":
            return tiles
        if order == "diag_first":
            return tiles[::-1]
    else:
        if order == "ascending":
            return list(range(nK))
        if order == "diag_first":
            start = min(max((r0 + Lk - Lq) // tk, 0), nK - 1)
            return list(range(start, nK)) + list(range(0, start))
    raise ValueError(f"unknown order {order!r}")


def stream_pass(s_tiles: list, v_tiles: list, thr: float, mode: str = "uniform",
                force: list | None = None) -> dict:
    """One streaming online-softmax pass with the skip test.

    ``s_tiles[t]``: fp64 scores [rows, keys_t] of the t-th visited tile
    (already multiplied by the softmax scale, -inf where a key is not
    visible); ``v_tiles[t]``: its value rows [keys_t, Dv].  ``force[t]``, when
    given, replaces the decision (bool, or a per-row bool array in per_row
    mode); the statistic delta is still recorded.

    Returns the normalised output [rows, Dv], lse [rows], the per-tile skip
    decisions and deltas, and the final m and l.
    """
    ln_thr = log_threshold(thr)
    rows = s_tiles[0].shape[0] if s_tiles else 0
    dv = v_tiles[0].shape[1] if v_tiles else 0
    m = np.full(rows, NEG_INF)
    l = np.zeros(rows)
    O = np.zeros((rows, dv))
    skips, deltas = [], []
    with np.errstate(invalid="ignore", over="ignore"):
        for t, (s, vt) in enumerate(zip(s_tiles, v_tiles)):
            tile_max = s.max(axis=1)
            delta_r = np.where(tile_max == NEG_INF, NEG_INF,
                               np.where(m == NEG_INF, math.inf, tile_max - m))
            if mode == "uniform":
                delta = float(delta_r.max())
                skip = np.full(rows, delta < ln_thr)
            elif mode == "per_row":
                delta = delta_r
                skip = delta_r < ln_thr
            else:
                raise ValueError(f"unknown mode {mode!r}")
            if force is not None:
                skip = np.broadcast_to(np.asarray(force[t], dtype=bool), (rows,)).copy()
            m_new = np.maximum(m, tile_max)
            # rescale factor for what is already accumulated; rows that have
            # seen no key yet hold l = O = 0, so any finite factor works there
            alpha = np.where(m_new == NEG_INF, 1.0, np.exp(m - m_new))
            keep = ~skip
            p = np.where(m_new[:, None] == NEG_INF, 0.0, np.exp(s - m_new[:, None]))
            l = alpha * l + np.where(keep, p.sum(axis=1), 0.0)
            O = alpha[:, None] * O + np.where(keep[:, None], p @ vt, 0.0)
            m = m_new
            skips.append(skip[0] if mode == "uniform" else skip)
            deltas.append(delta)
        has = l > 0
        out = np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
    return {"out": out, "lse": lse, "skip": skips, "delta": deltas, "m": m, "l": l}


def lse_combine(outs: np.ndarray, lses: np.ndarray) -> tuple:
    """Merge split results: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
    ``outs`` [S, rows, Dv], ``lses`` [S, rows].  Rows with every lse_s = -inf
    give O = 0 and lse = -inf."""
    with np.errstate(invalid="ignore", over="ignore"):
        mx = lses.max(axis=0)
        fin = mx > NEG_INF
        mxs = np.where(fin, mx, 0.0)
        w = np.exp(lses - mxs[None, :])
        tot = w.sum(axis=0)
        lse = np.where(fin, mxs + np.log(np.where(fin, tot, 1.0)), NEG_INF)
        wn = np.where(fin[None, :], w / np.where(fin, tot, 1.0)[None, :], 0.0)
        out = (wn[:, :, None] * outs).sum(axis=0)
    return out, lse


def prefill(q, k, v, scale: float, causal: bool, thr: float, *, tq: int = 128, tk: int = 128,
            mode: str = "uniform", order: str = "ascending", force_mask=None,
            blocks=None) -> dict:
    """Skip-softmax prefill.  q[B,Hq,Lq,D], k[B,Hkv,Lk,D], v[B,Hkv,Lk,Dv].

    Query head h reads KV head h // (Hq/Hkv).  ``force_mask`` (u8
    [B,Hq,nQ,nK], or [B,Hq,Lq,nK] in per_row mode) replaces the decisions of
    visited tiles.  ``blocks``: optional iterable of (b, h, i) query tiles to
    evaluate; rows of other tiles are left NaN and their mask entries 255.

    Returns ``out`` [B,Hq,Lq,Dv], ``lse`` [B,Hq,Lq], ``mask`` u8 [B,Hq,nQ,nK]
    (uniform mode) or ``row_mask`` u8 [B,Hq,Lq,nK] (per_row), ``delta``
    (same shape as the mask, NaN where not visited) and ``skip_fraction``.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    Dv = v.shape[-1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    nQ, nK = n_tiles(Lq, tq), n_tiles(Lk, tk)
    out = np.zeros((B, Hq, Lq, Dv))
    lse = np.full((B, Hq, Lq), NEG_INF)
    if mode == "uniform":
        mask = np.full((B, Hq, nQ, nK), MASK_UNVISITED, np.uint8)
        delta = np.full((B, Hq, nQ, nK), np.nan)
    else:
        mask = np.full((B, Hq, Lq, nK), MASK_UNVISITED, np.uint8)
        delta = np.full((B, Hq, Lq, nK), np.nan)
    if blocks is None:
        blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nQ)]
    else:
        blocks = list(blocks)
        out[:] = np.nan
        mask[:] = 255
    for b, h, i in blocks:
        hk = h // g
        rows = np.arange(i * tq, min((i + 1) * tq, Lq))
        tiles = visit_order(i, nK, Lq, Lk, causal, order, tq, tk)
        if mode == "uniform":
            mask[b, h, i, :] = MASK_UNVISITED
        else:
            mask[b, h, rows, :] = MASK_UNVISITED
        if not tiles:
            out[b, h, rows] = 0.0
            lse[b, h, rows] = NEG_INF
            continue
        s_tiles, v_tiles = [], []
        for j in tiles:
            keys = np.arange(j * tk, min((j + 1) * tk, Lk))
            s = scale * (q[b, h, rows] @ k[b, hk, keys].T)
            if causal:
                s[keys[None, :] > rows[:, None] + (Lk - Lq)] = NEG_INF
            s_tiles.append(s)
            v_tiles.append(v[b, hk, keys])
        force = None
        if force_mask is not None:
            fm = np.asarray(force_mask)
            if mode == "uniform":
                force = [fm[b, h, i, j] == MASK_SKIPPED for j in tiles]
            else:
                force = [fm[b, h, rows, j] == MASK_SKIPPED for j in tiles]
        res = stream_pass(s_tiles, v_tiles, thr, mode, force)
        out[b, h, rows] = res["out"]
        lse[b, h, rows] = res["lse"]
        for j, sk, dl in zip(tiles, res["skip"], res["delta"]):
            if mode == "uniform":
                mask[b, h, i, j] = MASK_SKIPPED if sk else MASK_COMPUTED
                delta[b, h, i, j] = dl
            else:
                mask[b, h, rows, j] = np.where(sk, MASK_SKIPPED, MASK_COMPUTED)
                delta[b, h, rows, j] = dl
    key = "mask" if mode == "uniform" else "row_mask"
    return {"out": out, "lse": lse, key: mask, "delta": delta,
            "skip_fraction": skip_fraction(mask)}


def decode(q, k, v, scale: float, thr: float, num_splits: int, *, tk: int = 128,
           mode: str = "uniform", force_mask=None, latent_dv: int | None = None,
           pairs=None) -> dict:
    """Split-KV skip-softmax decode for one query token per sequence.

    q[B,Hq,D], k[B,Hkv,Lk,D], v[B,Hkv,Lk,Dv]; with ``v is None`` the value
    rows are the first ``latent_dv`` columns of each key row (a shared latent
    cache).  The row block of a decision is the group of Hq/Hkv query heads
    reading one KV head.  ``pairs``: optional iterable of (b, hk) to evaluate
    (other outputs NaN, mask 255).

    Returns ``out`` [B,Hq,Dv], ``lse`` [B,Hq], ``mask`` u8 [B,Hkv,nK]
    (``row_mask`` u8 [B,Hq,nK] in per_row mode), ``delta``, the split ranges,
    the per-split partials ``part_out`` [S,B,Hq,Dv] / ``part_lse`` [S,B,Hq]
    and ``skip_fraction``.
    """
    q, k = to_f64(q), to_f64(k)
    B, Hq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    if v is None:
        if latent_dv is None or latent_dv > D:
            raise ValueError("latent decode needs latent_dv <= D")
        v = k[..., :latent_dv]
    else:
        v = to_f64(v)
    Dv = v.shape[-1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    nK = n_tiles(Lk, tk)
    splits = split_ranges(nK, num_splits)
    S = len(splits)
    out = np.zeros((B, Hq, Dv))
    lse = np.full((B, Hq), NEG_INF)
    part_out = np.zeros((S, B, Hq, Dv))
    part_lse = np.full((S, B, Hq), NEG_INF)
    if mode == "uniform":
        mask = np.full((B, Hkv, nK), MASK_UNVISITED, np.uint8)
        delta = np.full((B, Hkv, nK), np.nan)
    else:
        mask = np.full((B, Hq, nK), MASK_UNVISITED, np.uint8)
        delta = np.full((B, Hq, nK), np.nan)
    if pairs is None:
        pairs = [(b, hk) for b in range(B) for hk in range(Hkv)]
    else:
        pairs = list(pairs)
        out[:] = np.nan
        mask[:] = 255
    for b, hk in pairs:
        heads = slice(hk * g, (hk + 1) * g)
        qr = q[b, heads]
        scores = scale * (qr @ k[b, hk].T)  # [g, Lk]
        for si, (t0, t1) in enumerate(splits):
            tiles = list(range(t0, t1))
            s_tiles = [scores[:, j * tk:min((j + 1) * tk, Lk)] for j in tiles]
            v_tiles = [v[b, hk, j * tk:min((j + 1) * tk, Lk)] for j in tiles]
            force = None
            if force_mask is not None:
                fm = np.asarray(force_mask)
                if mode == "uniform":
                    force = [fm[b, hk, j] == MASK_SKIPPED for j in tiles]
                else:
                    force = [fm[b, heads, j] == MASK_SKIPPED for j in tiles]
            res = stream_pass(s_tiles, v_tiles, thr, mode, force)
            part_out[si, b, heads] = res["out"]
            part_lse[si, b, heads] = res["lse"]
            for j, sk, dl in zip(tiles, res["skip"], res["delta"]):
                if mode == "uniform":
                    mask[b, hk, j] = MASK_SKIPPED if sk else MASK_COMPUTED
                    delta[b, hk, j] = dl
                else:
                    mask[b, heads, j] = np.where(sk, MASK_SKIPPED, MASK_COMPUTED)
                    delta[b, heads, j] = dl
        o, ls = lse_combine(part_out[:, b, heads], part_lse[:, b, heads])
        out[b, heads] = o
        lse[b, heads] = ls
    key = "mask" if mode == "uniform" else "row_mask"
    return {"out": out, "lse": lse, key: mask, "delta": delta, "splits": splits,
            "part_out": part_out, "part_lse": part_lse, "skip_fraction": skip_fraction(mask)}


def skip_fraction(mask: np.ndarray) -> float:
    """#skipped / (#computed + #skipped) over visited tiles."""
    m = np.asarray(mask)
    sk = int((m == MASK_SKIPPED).sum())
    tot = sk + int((m == MASK_COMPUTED).sum())
    return sk / tot if tot else 0.0


def dense_prefill(q, k, v, scale: float, causal: bool) -> np.ndarray:
    """Plain two-pass softmax attention in fp64 (the exact, non-skipping result)."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Lq, _ = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, Lq, v.shape[-1]))
    rows = np.arange(Lq)[:, None]
    keys = np.arange(Lk)[None, :]
    hidden = keys > rows + (Lk - Lq) if causal else np.zeros((Lq, Lk), bool)
    with np.errstate(invalid="ignore"):
        for b in range(B):
            for h in range(Hq):
                s = scale * (q[b, h] @ k[b, h // g].T)
                s[hidden] = NEG_INF
                mx = s.max(axis=1, keepdims=True)
                seen = np.isfinite(mx)
                p = np.where(seen, np.exp(s - np.where(seen, mx, 0.0)), 0.0)
                den = p.sum(axis=1, keepdims=True)
                out[b, h] = np.where(seen, (p @ v[b, h // g]) / np.where(seen, den, 1.0), 0.0)
    return out


def dense_decode(q, k, v, scale: float, latent_dv: int | None = None) -> np.ndarray:
    """Plain two-pass softmax attention for one query token per sequence."""
    q, k = to_f64(q), to_f64(k)
    v = k[..., :latent_dv] if v is None else to_f64(v)
    B, Hq, _ = q.shape
    g = Hq // k.shape[1]
    out = np.zeros((B, Hq, v.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            s = scale * (k[b, h // g] @ q[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p @ v[b, h // g]) / p.sum()
    return out


def prefill_backward(q, k, v, do, scale: float, causal: bool, mask=None, *, tq: int = 128,
                     tk: int = 128) -> dict:
    """Gradients of the skip-softmax prefill with its skip decisions held fixed.

    The pages train models with the sparsity on (BLASST summary page,
    "Belangrijkste Bijdragen", the sparsity-aware training contribution) but
    print no backward pass;
    the plainest reading is the derivative of the forward output with the
    decisions replayed as constants (they are a threshold test, piecewise
    constant in the inputs).  With them fixed, row ``r`` of query tile ``i``
    attends by plain softmax (design page, "The online-softmax pass": the
    pass is exact over the keys it keeps) to the visible keys of the tiles
    ``j`` with ``mask[b, h, i, j] == 0``:

        P_r = softmax(scale * q_r K^T) over those keys,   O_r = P_r V
        dV += P^T dO,   dP = dO V^T,   D_r = dO_r . O_r,
        dS = P * (dP - D),   dQ = scale dS K,   dK += scale dS^T Q

    ``mask`` u8 [B,Hq,nQ,nK] (0 computed, 1 skipped, 2 not visited), as the
    forward wrote it; ``None`` keeps every visible tile (dense attention).
    Query head h reads (and sends gradient to) KV head h // (Hq/Hkv).
    Returns ``dq`` [B,Hq,Lq,D], ``dk`` [B,Hkv,Lk,D], ``dv`` [B,Hkv,Lk,Dv],
    and the forward ``out``, ``lse`` (ln of the row's kept exponential sum,
    -inf for a row with no kept key) and ``D`` = rowsum(dO * O).
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, Hq, Lq, Dq = q.shape
    _, Hkv, Lk, _ = k.shape
    Dv = v.shape[-1]
    g = Hq // Hkv
    nQ, nK = n_tiles(Lq, tq), n_tiles(Lk, tk)
    m = None if mask is None else np.asarray(mask)
    dq = np.zeros_like(q)
    dk = np.zeros((B, Hkv, Lk, Dq))
    dv = np.zeros((B, Hkv, Lk, Dv))
    out = np.zeros((B, Hq, Lq, Dv))
    lse = np.full((B, Hq, Lq), NEG_INF)
    dvec = np.zeros((B, Hq, Lq))
    keys_all = np.arange(Lk)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(nQ):
                rows = np.arange(i * tq, min((i + 1) * tq, Lq))
                kept = np.zeros(Lk, bool)
                for j in range(nK):
                    if m is None or m[b, h, i, j] == MASK_COMPUTED:
                        kept[j * tk:(j + 1) * tk] = True
                vis = np.broadcast_to(kept[None, :], (len(rows), Lk)).copy()
                if causal:
                    vis &= keys_all[None, :] <= rows[:, None] + (Lk - Lq)
                s = scale * (q[b, h, rows] @ k[b, hk].T)
                s = np.where(vis, s, NEG_INF)
                mx = s.max(axis=1, keepdims=True)
                seen = np.isfinite(mx)[:, 0]
                p = np.zeros_like(s)
                if seen.any():
                    e = np.exp(s[seen] - mx[seen])
                    den = e.sum(axis=1, keepdims=True)
                    p[seen] = e / den
                    lse[b, h, rows[seen]] = (mx[seen] + np.log(den))[:, 0]
                o = p @ v[b, hk]
                out[b, h, rows] = o
                dor = do[b, h, rows]
                dp = dor @ v[b, hk].T
                d = (dor * o).sum(axis=1)
                ds = p * (dp - d[:, None])
                dvec[b, h, rows] = d
                dv[b, hk] += p.T @ dor
                dq[b, h, rows] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ q[b, h, rows])
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse, "D": dvec}
