"""GPU parity: the HIP kernels against the fp64 oracle, through the C ABI.

Masks are graded with the margin rule (tiles within 1e-3 relative of the
threshold may flip; every other tile must match; >= 99.9 % agreement).
Outputs are graded against the oracle re-run with the GPU's own mask forced:
rel-L2 <= 1e-2 for bf16 inputs, <= 1e-5 for the fp32 debug path.  Small cases
span several tiles with ragged tails and run the oracle on everything; the
full-size cases run the GPU on the whole call and the oracle on sampled
query tiles / (batch, KV head) pairs.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.grading import ROW_FACTOR, grade_masks, max_row_rel_l2, rel_l2
from synth import WORKLOADS, clustered_decode, clustered_prefill, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def log(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- prefill helpers

def gpu_prefill(ss, x, scale, causal, thr, order):
    q, k, v = (x[n].cuda() for n in "qkv")
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    mask = torch.full(ss.mask_shape_prefill(B, Hq, Lq, Lk), 255, dtype=torch.uint8, device="cuda")
    out = ss.ss_attn_prefill_ex(q, k, v, scale=scale, causal=causal, threshold=thr,
                                skip_mask=mask, order=order)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), mask.cpu().numpy()


def check_prefill(ss, x, scale, causal, thr, order, dtype, blocks=None, name=""):
    out, mask = gpu_prefill(ss, x, scale, causal, thr, order)
    ref = oracle.prefill(x["q"], x["k"], x["v"], scale, causal, thr, order=order, blocks=blocks)
    B, Hq, Lq, _ = x["q"].shape
    if blocks is None:
        sel_mask, sel_rows = None, np.ones((B, Hq, Lq), bool)
    else:
        sel_mask = np.zeros(ref["mask"].shape, bool)
        sel_rows = np.zeros((B, Hq, Lq), bool)
        for b, h, i in blocks:
            sel_mask[b, h, i] = True
            sel_rows[b, h, i * 128:(i + 1) * 128] = True
    assert np.isin(mask, (0, 1, 2)).all(), "unwritten mask entries"
    gr = grade_masks(mask, ref["mask"], ref["delta"], thr, sel_mask)
    assert gr["ok"], f"{name}: mask {gr}"
    forced = oracle.prefill(x["q"], x["k"], x["v"], scale, causal, thr, order=order,
                            force_mask=np.where(sel_mask if sel_mask is not None else True, mask, 0),
                            blocks=blocks)
    err = rel_l2(out[sel_rows], forced["out"][sel_rows])
    row = max_row_rel_l2(out[sel_rows], forced["out"][sel_rows])
    own = rel_l2(out[sel_rows], ref["out"][sel_rows])
    visited = np.isin(mask, (0, 1)) if sel_mask is None else (np.isin(mask, (0, 1)) & sel_mask)
    skip = float((mask[visited] == 1).mean()) if visited.any() else 0.0
    log(f"[prefill {name}] thr={thr} order={order} skip={skip:.3f} rel-L2 vs forced={err:.2e} "
        f"vs oracle mask={own:.2e} worst row={row:.2e} mask agreement={gr['agreement']:.4f} "
        f"near={gr['near']}")
    assert err <= TOL[dtype], f"{name}: rel-L2 {err}"
    assert row <= ROW_FACTOR * TOL[dtype], f"{name}: worst row rel-L2 {row}"
    assert np.isfinite(out[sel_rows]).all()
    return out, mask


PREFILL_CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, causal, order, r, thr
    ("causal_gqa_ragged", 1, 4, 2, 1000, 1000, 128, True, "ascending", 9.0, 0.05),
    ("causal_gqa_diag", 1, 4, 2, 1000, 1000, 128, True, "diag_first", 9.0, 0.05),
    ("lq_below_lk", 2, 2, 1, 700, 1300, 128, True, "diag_first", 9.0, 0.2),
    ("lq_above_lk", 1, 2, 2, 900, 400, 64, True, "ascending", 9.0, 0.1),
    ("noncausal_d64_diag", 1, 3, 1, 1000, 1000, 64, False, "diag_first", 9.0, 0.01),
    ("d64_gqa_pairs", 2, 8, 2, 700, 900, 64, False, "ascending", 9.0, 0.05),
    ("causal_gqa_group6", 1, 6, 1, 520, 520, 128, True, "diag_first", 9.0, 0.05),
    ("noncausal_ragged", 1, 2, 1, 513, 777, 128, False, "ascending", 9.0, 0.3),
    ("thr_above_one", 1, 2, 1, 513, 777, 128, False, "ascending", 3.0, 2.0),
    ("thr_one", 1, 2, 2, 640, 640, 128, True, "diag_first", 3.0, 1.0),
    ("dense", 1, 4, 1, 1000, 1000, 128, True, "ascending", 3.0, 0.0),
    ("single_tile", 1, 1, 1, 100, 100, 64, True, "ascending", 3.0, 0.5),
    ("one_query_row", 1, 1, 1, 1, 300, 128, True, "ascending", 9.0, 0.1),
    # odd group sizes run two neighbouring query tiles of one head per
    # workgroup over a shared key stream: odd tile counts, Lq != Lk, both
    # orders, causal and not
    ("mha_causal_diag_lq_below_lk", 1, 2, 2, 650, 1100, 128, True, "diag_first", 9.0, 0.1),
    ("mha_noncausal_diag_lq_below_lk", 1, 3, 3, 700, 1300, 64, False, "diag_first", 9.0, 0.05),
    ("mha_noncausal_diag_lq_above_lk", 1, 1, 1, 1300, 700, 128, False, "diag_first", 9.0, 0.05),
    ("mha_causal_asc_odd_tiles", 1, 1, 1, 1100, 1100, 128, True, "ascending", 9.0, 0.1),
    ("gqa3_causal_diag_odd_tiles", 1, 6, 2, 1100, 1100, 128, True, "diag_first", 9.0, 0.05),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_small(ss, case, dtype):
    name, B, Hq, Hkv, Lq, Lk, D, causal, order, r, thr = case
    x = clustered_prefill(zlib.crc32(name.encode()) % 10000, B, Hq, Hkv, Lq, Lk, D, D, 16, r, "tile", dtype=dtype)
    check_prefill(ss, x, 1 / math.sqrt(D), causal, thr, order, dtype, name=f"{name}/{dtype}")


@pytest.mark.parametrize("thr", [0.0, 1e-4, 1e-3])
def test_prefill_tiny_f32_workload(ss, thr):
    """Tiny non-causal fp32 case (B1 H1 L1024 D64, scale 1/8, 8 centroids r=3)."""
    w = WORKLOADS["tiny_f32"]
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in "qkv")
    mask = torch.empty(ss.mask_shape_prefill(1, 1, 1024, 1024), dtype=torch.uint8, device="cuda")
    out = ss.ss_attn_prefill_f32(q, k, v, scale=w.scale, threshold=thr, skip_mask=mask)
    torch.cuda.synchronize()
    ref = oracle.prefill(x["q"], x["k"], x["v"], w.scale, False, thr)
    gr = grade_masks(mask.cpu().numpy(), ref["mask"], ref["delta"], thr)
    assert gr["ok"], gr
    err = rel_l2(out.cpu().numpy(), ref["out"])
    assert max_row_rel_l2(out.cpu().numpy(), ref["out"]) <= ROW_FACTOR * 1e-5
    dense = oracle.dense_prefill(x["q"], x["k"], x["v"], w.scale, False)
    log(f"[tiny_f32] thr={thr} skip={ref['skip_fraction']:.3f} rel-L2={err:.2e} "
        f"vs dense={rel_l2(out.cpu().numpy(), dense):.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("thr", [1e-3, 1e-2, 0.1, 1.0])
@pytest.mark.parametrize("name", ["tiny_tile_f32", "tiny_tile_bf16"])
def test_prefill_tiny_tile_workloads(ss, name, thr):
    w = WORKLOADS[name]
    x = make_inputs(w)
    check_prefill(ss, x, w.scale, w.causal, thr, "ascending", w.dtype, name=name)


@pytest.mark.parametrize("thr,order", [(0.0, "ascending"), (0.5, "ascending"),
                                       (0.5, "diag_first")])
def test_prefill_gqa_16k_full_size_sampled(ss, thr, order):
    """Causal GQA prefill at full size (B1 Hq32 Hkv8 L16384 D128); the oracle
    checks 9 sampled query tiles across heads and positions."""
    w = WORKLOADS["gqa_prefill_16k"]
    x = make_inputs(w)
    blocks = [(0, h, i) for h in (0, 13, 31) for i in (0, 37, 127)]
    check_prefill(ss, x, w.scale, True, thr, order, "bf16", blocks=blocks, name=w.name)


def test_prefill_video_dit_full_size_sampled(ss):
    """Non-causal video-DiT prefill at full size (H24 L32760 D128, ragged last tile)."""
    w = WORKLOADS["video_dit_32760"]
    x = make_inputs(w)
    thr = 3.0 / w.Lk
    blocks = [(0, h, i) for h in (0, 23) for i in (0, 100, 255)]
    for order in ("ascending", "diag_first"):
        check_prefill(ss, x, w.scale, False, thr, order, "bf16", blocks=blocks, name=w.name)


# --------------------------------------------------------------------------- decode

def gpu_decode(ss, x, scale, thr, S, latent_dv=None, mode="chained"):
    """Run the decode through the C ABI with a zeroed workspace; returns the
    output, the mask and the look-back timeout count left in the workspace."""
    q, k = x["q"].cuda(), x["k"].cuda()
    v = None if x["v"] is None else x["v"].cuda()
    B, Hq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    Dv = latent_dv or v.shape[3]
    mask = torch.full(ss.mask_shape_decode(B, Hkv, Lk), 255, dtype=torch.uint8, device="cuda")
    nbytes = ss.ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, S)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = ss.ss_attn_decode_ex(q, k, v, dv=latent_dv, scale=scale, threshold=thr, num_splits=S,
                               split_mode=mode, skip_mask=mask, workspace=ws)
    torch.cuda.synchronize()
    timeouts = int(ws[nbytes - 256:nbytes - 252].view(torch.int32).item())
    return out.float().cpu().numpy(), mask.cpu().numpy(), timeouts


def check_decode(ss, x, scale, thr, S, pairs=None, latent_dv=None, name="", mode="chained"):
    out, mask, timeouts = gpu_decode(ss, x, scale, thr, S, latent_dv, mode)
    assert timeouts == 0, f"{name}: {timeouts} look-back waits gave up"
    B, Hq, D = x["q"].shape
    Hkv, Lk = x["k"].shape[1], x["k"].shape[2]
    Dv = latent_dv or x["v"].shape[3]
    if mode == "chained":
        S_ref = 1  # chained splits decide as one streaming pass
    else:
        S_ref = S or ss.ss_decode_num_splits(B, Hq, Hkv, Lk, D, Dv)
    ref = oracle.decode(x["q"], x["k"], x["v"], scale, thr, S_ref, latent_dv=latent_dv,
                        pairs=pairs)
    g = Hq // Hkv
    if pairs is None:
        sel_mask, sel_rows = None, np.ones((B, Hq), bool)
    else:
        sel_mask = np.zeros(ref["mask"].shape, bool)
        sel_rows = np.zeros((B, Hq), bool)
        for b, hk in pairs:
            sel_mask[b, hk] = True
            sel_rows[b, hk * g:(hk + 1) * g] = True
    assert np.isin(mask, (0, 1)).all(), "unwritten decode mask entries"
    gr = grade_masks(mask, ref["mask"], ref["delta"], thr, sel_mask)
    assert gr["ok"], f"{name}: mask {gr}"
    forced = oracle.decode(x["q"], x["k"], x["v"], scale, thr, S_ref, latent_dv=latent_dv,
                           pairs=pairs, force_mask=mask)
    err = rel_l2(out[sel_rows], forced["out"][sel_rows])
    row = max_row_rel_l2(out[sel_rows], forced["out"][sel_rows])
    own = rel_l2(out[sel_rows], ref["out"][sel_rows])
    sm = mask if sel_mask is None else mask[sel_mask]
    log(f"[decode {name}] mode={mode} thr={thr} splits={S} skip={float((sm == 1).mean()):.3f} "
        f"rel-L2 vs forced={err:.2e} vs oracle mask={own:.2e} worst row={row:.2e} "
        f"agreement={gr['agreement']:.4f}")
    assert err <= TOL["bf16"], f"{name}: rel-L2 {err}"
    assert row <= ROW_FACTOR * TOL["bf16"], f"{name}: worst row rel-L2 {row}"
    return out, mask


DECODE_CASES = [
    # name, B, Hq, Hkv, Lk, D, S, r, thr
    ("gqa4_auto", 2, 8, 2, 5000, 128, 0, 9.0, 0.05),
    ("mha_d64", 3, 4, 4, 777, 64, 2, 9.0, 0.3),
    ("mqa8_thr1", 1, 8, 1, 3000, 128, 5, 9.0, 1.0),
    ("gqa8_one_split", 2, 16, 2, 4100, 128, 1, 9.0, 0.01),
    ("one_tile", 1, 2, 1, 128, 64, 1, 3.0, 0.5),
    ("dense", 2, 4, 2, 2000, 128, 3, 3.0, 0.0),
    ("thr_above_one", 1, 4, 2, 3333, 64, 4, 3.0, 2.0),
    ("one_key", 1, 2, 2, 1, 128, 1, 3.0, 0.1),
    ("gqa2_many_splits", 1, 4, 2, 2500, 128, 99, 9.0, 0.05),
    ("g1_long_chain", 1, 2, 2, 20000, 128, 0, 9.0, 0.02),
    # other group sizes: 3..7 query heads per KV head, and multi-query
    # attention with 16 or 32 heads on one KV head
    ("gqa3_d64", 2, 6, 2, 3000, 64, 0, 9.0, 0.05),
    ("gqa5_ragged", 1, 10, 2, 2777, 128, 3, 9.0, 0.1),
    ("mqa6", 2, 6, 1, 5000, 128, 0, 9.0, 0.05),
    ("gqa7", 1, 14, 2, 1500, 128, 2, 9.0, 0.2),
    ("mqa16", 2, 16, 1, 6000, 128, 0, 9.0, 0.05),
    ("mqa16_dense_one_split", 1, 16, 1, 1000, 128, 1, 3.0, 0.0),
    ("mqa32", 2, 32, 1, 6000, 128, 0, 9.0, 0.05),
    ("mqa32_d64_thr1", 1, 32, 1, 3000, 64, 4, 9.0, 1.0),
    ("mqa32_long_chain", 1, 32, 1, 20000, 128, 0, 9.0, 0.02),
]


@pytest.mark.parametrize("mode", ["chained", "independent"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small(ss, case, mode):
    name, B, Hq, Hkv, Lk, D, S, r, thr = case
    x = clustered_decode(zlib.crc32(name.encode()) % 10000, B, Hq, Hkv, Lk, D, D, 16, r)
    check_decode(ss, x, 1 / math.sqrt(D), thr, S, name=name, mode=mode)


@pytest.mark.parametrize("thr,mode", [(0.0, "chained"), (0.6, "chained"), (0.95, "independent")])
def test_decode_gqa_32k_full_size(ss, thr, mode):
    """GQA decode at full size (B16 Hq32 Hkv8 Lk32768 D128) with the automatic
    split count; the oracle checks 24 sampled (batch, KV head) pairs."""
    w = WORKLOADS["gqa_decode_32k"]
    x = make_inputs(w)
    rng = np.random.default_rng(0)
    pairs = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 16, 24), rng.integers(0, 8, 24))})
    check_decode(ss, x, w.scale, thr, 0, pairs=pairs, name=w.name, mode=mode)


MLA_CASES = [
    # name, B, Hq, Lk, S, r, thr  (one latent head: D = 576, value = first 512 columns)
    ("mla128_auto", 2, 128, 3000, 0, 9.0, 0.05),
    ("mla64_splits", 1, 64, 2000, 3, 9.0, 0.1),
    ("mla128_dense", 1, 128, 1500, 2, 3.0, 0.0),
    ("mla128_thr1", 1, 128, 2500, 4, 9.0, 1.0),
    ("mla128_thr_above_one", 1, 128, 1000, 2, 3.0, 2.0),
    ("mla128_one_key", 1, 128, 1, 1, 3.0, 0.1),
    ("mla128_many_splits", 1, 128, 2500, 99, 9.0, 0.05),
    ("mla128_long_chain", 1, 128, 20000, 0, 9.0, 0.02),
    ("mla128_share_out", 2, 128, 8192, 2, 9.0, 0.05),  # 32 tiles per sub-split: shared out
    ("mla64_share_out_ragged", 1, 64, 9000, 3, 9.0, 0.05),
]


@pytest.mark.parametrize("mode", ["chained", "independent"])
@pytest.mark.parametrize("case", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_decode_mla_small(ss, case, mode):
    name, B, Hq, Lk, S, r, thr = case
    x = clustered_decode(zlib.crc32(name.encode()) % 10000, B, Hq, 1, Lk, 576, 512, 16, r,
                         latent=True)
    check_decode(ss, x, 1 / 24, thr, S, latent_dv=512, name=name, mode=mode)


MLA_STREAM_CASES = [
    # name, B, Hq, Lk, S, r, thr: every split a whole chain of at most 64
    # tiles, so the decode runs as one streaming pass per split
    ("mla128_one_chain_64_tiles", 2, 128, 8192, 1, 9.0, 0.05),
    ("mla64_one_chain_ragged", 1, 64, 8192 - 37, 1, 9.0, 0.1),
    ("mla128_four_chains", 3, 128, 5000, 4, 9.0, 0.05),
    ("mla128_chains_thr1", 1, 128, 6000, 2, 9.0, 1.0),
    ("mla64_chains_thr2", 2, 64, 4000, 3, 3.0, 2.0),
    ("mla128_chains_dense_like", 1, 128, 3000, 2, 3.0, 1e-4),
]


@pytest.mark.parametrize("case", MLA_STREAM_CASES, ids=[c[0] for c in MLA_STREAM_CASES])
def test_decode_mla_stream(ss, case):
    name, B, Hq, Lk, S, r, thr = case
    x = clustered_decode(zlib.crc32(name.encode()) % 10000, B, Hq, 1, Lk, 576, 512, 16, r,
                         latent=True)
    check_decode(ss, x, 1 / 24, thr, S, latent_dv=512, name=name, mode="independent")
    if S == 1:
        check_decode(ss, x, 1 / 24, thr, S, latent_dv=512, name=name, mode="chained")


def test_decode_mla_stream_score_jump(ss):
    """One chain of 64 tiles whose tile 40 scores about 60 nats above the rest
    for every head: far beyond the range the streaming pass lets its
    exponent reference trail the running max, so the pass runs again with
    each head's max over the chain as reference.  The output is then carried
    almost entirely by tile 40."""
    x = clustered_decode(77, 1, 128, 1, 8192, 576, 512, 16, 9.0, latent=True)
    u = x["q"][0].float().mean(0)
    alpha = 60.0 * 24 / float(u @ u)
    k = x["k"].float()
    k[0, 0, 40 * 128:41 * 128] = 0.1 * k[0, 0, 40 * 128:41 * 128] + alpha * u
    x["k"] = k.to(torch.bfloat16)
    _, mask = check_decode(ss, x, 1 / 24, 0.05, 1, latent_dv=512, name="mla_score_jump",
                           mode="independent")
    assert mask[0, 0, 40] == 0


@pytest.mark.parametrize("thr,mode", [(0.0, "chained"), (0.3, "chained"), (0.5, "independent")])
def test_decode_mla_16k_full_size(ss, thr, mode):
    """Latent decode at full size (B8 Hq128 Lk16384, 576-wide latent rows,
    value = first 512 columns) with the automatic split count; the oracle
    checks three sampled batch entries."""
    w = WORKLOADS["mla_decode_16k"]
    x = make_inputs(w)
    check_decode(ss, x, w.scale, thr, 0, pairs=[(0, 0), (3, 0), (7, 0)], latent_dv=512,
                 name=w.name, mode=mode)


def test_decode_mla_128k_full_size(ss):
    """Latent decode at the 131072-key size the latent timing uses (B8 Hq128),
    chained splits, at a threshold near its 70 % skip point, so the share-out
    of kept tiles over each sequence's workgroups runs at its real shape; the
    oracle checks one sampled sequence."""
    w = WORKLOADS["mla_decode_128k"]
    x = make_inputs(w)
    _, mask = check_decode(ss, x, w.scale, 0.9866, 0, pairs=[(5, 0)], latent_dv=512,
                           name=w.name, mode="chained")
    assert 0.6 < float((mask[5, 0] == 1).mean()) < 0.8


# --------------------------------------------------------------------------- determinism

def test_repeat_runs_are_bitwise_identical(ss):
    x = clustered_prefill(5, 1, 4, 2, 1000, 1000, 128, 128, 16, 9.0, "tile")
    a = gpu_prefill(ss, x, 1 / math.sqrt(128), True, 0.05, "diag_first")
    b = gpu_prefill(ss, x, 1 / math.sqrt(128), True, 0.05, "diag_first")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    d = clustered_decode(6, 2, 8, 2, 5000, 128, 128, 16, 9.0)
    for mode in ("chained", "independent"):
        c1 = gpu_decode(ss, d, 1 / math.sqrt(128), 0.05, 0, mode=mode)
        c2 = gpu_decode(ss, d, 1 / math.sqrt(128), 0.05, 0, mode=mode)
        assert np.array_equal(c1[0], c2[0]) and np.array_equal(c1[1], c2[1])
