"""GPU parity of per-row skip decisions (granularity "row") against the oracle.

In per-row mode every query row takes the skip test alone (the oracle's
``mode="per_row"``): a row that fails it adds nothing from the tile, while
the tile itself -- its exponentials, its P.V, in decode its V read -- is
skipped only where every row of the row block fails.  Checked through the C
ABI on the bf16 and fp32 prefill and on the separate-V decode:

* the per-row mask against the oracle's row mask under the margin rule;
* the tile mask the kernel writes equals "every row of the block skipped"
  read off its own row mask, and equals the tile mask of the default
  (per-tile) mode on the same inputs bit for bit -- the running maxima do not
  depend on the mode, so neither does the tile rule;
* the output against the oracle re-run with the GPU's row mask forced
  (rel-L2 <= 1e-2 bf16, <= 1e-5 fp32).

Queries use the generator's "row" mode (every query row near its own random
centroid), where rows of one tile disagree most.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.grading import ROW_FACTOR, grade_masks, max_row_rel_l2, rel_l2
from synth import WORKLOADS, clustered_decode, clustered_prefill, make_inputs
from tests.test_parity_gpu import TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


# --------------------------------------------------------------------------- prefill

def run_prefill(ss, x, scale, causal, thr, order, granularity):
    q, k, v = (x[n].cuda() for n in "qkv")
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    tmask = torch.full(ss.mask_shape_prefill(B, Hq, Lq, Lk), 255, dtype=torch.uint8,
                       device="cuda")
    rmask = None
    if granularity == "row":
        rmask = torch.full(ss.row_mask_shape_prefill(B, Hq, Lq, Lk), 255, dtype=torch.uint8,
                           device="cuda")
    out = ss.ss_attn_prefill_ex(q, k, v, scale=scale, causal=causal, threshold=thr,
                                skip_mask=tmask, order=order, granularity=granularity,
                                row_mask=rmask)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), tmask.cpu().numpy(),
            None if rmask is None else rmask.cpu().numpy())


def tile_mask_from_rows(rmask, Lq):
    """[B,H,Lq,nK] row mask -> [B,H,nQ,nK]: 2 unvisited, 1 every row skipped, else 0."""
    B, H, _, nK = rmask.shape
    nQ = -(-Lq // 128)
    t = np.zeros((B, H, nQ, nK), np.uint8)
    for i in range(nQ):
        rows = rmask[:, :, i * 128:min((i + 1) * 128, Lq)]
        t[:, :, i] = np.where((rows == 2).all(axis=2), 2, np.where((rows == 1).all(axis=2), 1, 0))
    return t


def check_prefill_rows(ss, x, scale, causal, thr, order, dtype, name, blocks=None):
    out, tmask, rmask = run_prefill(ss, x, scale, causal, thr, order, "row")
    _, tmask_uniform, _ = run_prefill(ss, x, scale, causal, thr, order, "tile")
    B, Hq, Lq, _ = x["q"].shape
    assert np.array_equal(tmask, tmask_uniform), f"{name}: tile masks differ between modes"
    assert np.array_equal(tmask, tile_mask_from_rows(rmask, Lq)), f"{name}: tile vs row mask"
    ref = oracle.prefill(x["q"], x["k"], x["v"], scale, causal, thr, order=order,
                         mode="per_row", blocks=blocks)
    if blocks is None:
        sel = np.ones(rmask.shape, bool)
    else:
        sel = np.zeros(rmask.shape, bool)
        for b, h, i in blocks:
            sel[b, h, i * 128:(i + 1) * 128] = True
    sel_rows = sel[..., 0]
    assert np.isin(rmask[sel], (0, 1, 2)).all(), f"{name}: unwritten row-mask entries"
    gr = grade_masks(rmask, ref["row_mask"], ref["delta"], thr, sel)
    assert gr["ok"], f"{name}: row mask {gr}"
    forced = oracle.prefill(x["q"], x["k"], x["v"], scale, causal, thr, order=order,
                            mode="per_row", force_mask=np.where(sel, rmask, 0), blocks=blocks)
    err = rel_l2(out[sel_rows], forced["out"][sel_rows])
    vis_r = np.isin(rmask, (0, 1)) & sel
    vis_t = np.isin(tmask, (0, 1))
    log(f"[prefill rows {name}] thr={thr} order={order} row skip="
        f"{float((rmask[vis_r] == 1).mean()) if vis_r.any() else 0.0:.3f} tile skip="
        f"{float((tmask[vis_t] == 1).mean()) if vis_t.any() else 0.0:.3f} rel-L2 vs forced="
        f"{err:.2e} agreement={gr['agreement']:.4f} near={gr['near']}")
    assert err <= TOL[dtype], f"{name}: rel-L2 {err}"
    row = max_row_rel_l2(out[sel_rows], forced["out"][sel_rows])
    assert row <= ROW_FACTOR * TOL[dtype], f"{name}: worst row rel-L2 {row}"
    assert np.isfinite(out[sel_rows]).all()


PREFILL_ROW_CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, causal, order, r, thr
    ("causal_gqa_ragged", 1, 4, 2, 1000, 1000, 128, True, "ascending", 9.0, 0.05),
    ("causal_diag", 1, 2, 1, 900, 900, 128, True, "diag_first", 9.0, 0.2),
    ("lq_below_lk", 2, 2, 1, 700, 1300, 64, True, "diag_first", 9.0, 0.2),
    ("lq_above_lk", 1, 2, 2, 900, 400, 64, True, "ascending", 9.0, 0.1),
    ("noncausal_ragged", 1, 2, 1, 513, 777, 128, False, "ascending", 9.0, 0.3),
    ("d64_gqa_pairs", 2, 8, 2, 700, 900, 64, False, "diag_first", 9.0, 0.05),
    ("thr_one", 1, 2, 2, 640, 640, 128, True, "diag_first", 3.0, 1.0),
    ("thr_above_one", 1, 2, 1, 513, 777, 128, False, "ascending", 3.0, 2.0),
    ("dense", 1, 2, 1, 600, 600, 128, True, "ascending", 3.0, 0.0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", PREFILL_ROW_CASES, ids=[c[0] for c in PREFILL_ROW_CASES])
def test_prefill_per_row(ss, case, dtype):
    name, B, Hq, Hkv, Lq, Lk, D, causal, order, r, thr = case
    x = clustered_prefill(zlib.crc32(name.encode()) % 10000 + 7, B, Hq, Hkv, Lq, Lk, D, D, 16, r,
                          "row", dtype=dtype)
    check_prefill_rows(ss, x, 1 / math.sqrt(D), causal, thr, order, dtype, f"{name}/{dtype}")


def test_prefill_per_row_16k_full_size_sampled(ss):
    """Causal GQA prefill (B1 Hq32 Hkv8 L16384 D128), per-row, 6 sampled tiles."""
    w = WORKLOADS["gqa_prefill_16k"]
    x = make_inputs(w)
    blocks = [(0, h, i) for h in (3, 30) for i in (0, 64, 127)]
    check_prefill_rows(ss, x, w.scale, True, 0.5, "diag_first", "bf16", w.name, blocks=blocks)


# --------------------------------------------------------------------------- decode

def run_decode(ss, x, scale, thr, S, mode, granularity):
    q, k, v = (x[n].cuda() for n in "qkv")
    B, Hq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    tmask = torch.full(ss.mask_shape_decode(B, Hkv, Lk), 255, dtype=torch.uint8, device="cuda")
    rmask = None
    if granularity == "row":
        rmask = torch.full(ss.row_mask_shape_decode(B, Hq, Lk), 255, dtype=torch.uint8,
                           device="cuda")
    nbytes = ss.ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, D, S)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = ss.ss_attn_decode_ex(q, k, v, scale=scale, threshold=thr, num_splits=S,
                               split_mode=mode, skip_mask=tmask, workspace=ws,
                               granularity=granularity, row_mask=rmask)
    torch.cuda.synchronize()
    timeouts = int(ws[nbytes - 256:nbytes - 252].view(torch.int32).item())
    return (out.float().cpu().numpy(), tmask.cpu().numpy(),
            None if rmask is None else rmask.cpu().numpy(), timeouts)


def check_decode_rows(ss, x, scale, thr, S, mode, name, pairs=None):
    out, tmask, rmask, timeouts = run_decode(ss, x, scale, thr, S, mode, "row")
    _, tmask_uniform, _, _ = run_decode(ss, x, scale, thr, S, mode, "tile")
    assert timeouts == 0, f"{name}: {timeouts} look-back waits gave up"
    B, Hq, D = x["q"].shape
    Hkv, Lk = x["k"].shape[1], x["k"].shape[2]
    g = Hq // Hkv
    assert np.array_equal(tmask, tmask_uniform), f"{name}: tile masks differ between modes"
    grouped = rmask.reshape(B, Hkv, g, -1)
    assert np.array_equal(tmask, np.where((grouped == 1).all(axis=2), 1, 0)), \
        f"{name}: tile vs row mask"
    S_ref = 1 if mode == "chained" else (S or ss.ss_decode_num_splits(B, Hq, Hkv, Lk, D, D))
    ref = oracle.decode(x["q"], x["k"], x["v"], scale, thr, S_ref, mode="per_row", pairs=pairs)
    if pairs is None:
        sel_rows = np.ones((B, Hq), bool)
    else:
        sel_rows = np.zeros((B, Hq), bool)
        for b, hk in pairs:
            sel_rows[b, hk * g:(hk + 1) * g] = True
    sel = np.broadcast_to(sel_rows[..., None], rmask.shape)
    assert np.isin(rmask, (0, 1)).all(), f"{name}: unwritten row-mask entries"
    gr = grade_masks(rmask, ref["row_mask"], ref["delta"], thr, sel)
    assert gr["ok"], f"{name}: row mask {gr}"
    forced = oracle.decode(x["q"], x["k"], x["v"], scale, thr, S_ref, mode="per_row",
                           pairs=pairs, force_mask=rmask)
    err = rel_l2(out[sel_rows], forced["out"][sel_rows])
    log(f"[decode rows {name}] mode={mode} thr={thr} S={S} row skip="
        f"{float((rmask[sel] == 1).mean()):.3f} tile skip={float((tmask == 1).mean()):.3f} "
        f"rel-L2 vs forced={err:.2e} agreement={gr['agreement']:.4f}")
    assert err <= TOL["bf16"], f"{name}: rel-L2 {err}"
    row = max_row_rel_l2(out[sel_rows], forced["out"][sel_rows])
    assert row <= ROW_FACTOR * TOL["bf16"], f"{name}: worst row rel-L2 {row}"


DECODE_ROW_CASES = [
    # name, B, Hq, Hkv, Lk, D, S, r, thr
    ("gqa4_auto", 2, 8, 2, 5000, 128, 0, 9.0, 0.05),
    ("gqa8_d64", 2, 16, 2, 3000, 64, 3, 9.0, 0.1),
    ("gqa2_many_splits", 1, 4, 2, 2500, 128, 40, 9.0, 0.05),
    ("mha", 2, 4, 4, 1500, 128, 2, 9.0, 0.3),
    ("thr_above_one", 1, 8, 2, 2000, 128, 3, 3.0, 2.0),
    ("g1_long_chain", 1, 2, 2, 20000, 128, 0, 9.0, 0.02),
    ("gqa6", 2, 12, 2, 3000, 128, 0, 9.0, 0.05),
    ("mqa32", 1, 32, 1, 4000, 128, 0, 9.0, 0.05),
]


@pytest.mark.parametrize("mode", ["chained", "independent"])
@pytest.mark.parametrize("case", DECODE_ROW_CASES, ids=[c[0] for c in DECODE_ROW_CASES])
def test_decode_per_row(ss, case, mode):
    name, B, Hq, Hkv, Lk, D, S, r, thr = case
    x = clustered_decode(zlib.crc32(name.encode()) % 10000 + 11, B, Hq, Hkv, Lk, D, D, 16, r,
                         sigma=2.0)
    check_decode_rows(ss, x, 1 / math.sqrt(D), thr, S, mode, name)


def test_decode_per_row_32k_full_size_sampled(ss):
    """GQA decode at full size (B16 Hq32 Hkv8 Lk32768 D128), per-row, chained,
    the oracle on 12 sampled (batch, KV head) pairs."""
    w = WORKLOADS["gqa_decode_32k"]
    x = make_inputs(w)
    rng = np.random.default_rng(5)
    pairs = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 12), rng.integers(0, 8, 12))})
    check_decode_rows(ss, x, w.scale, 0.7, 0, "chained", w.name, pairs=pairs)
