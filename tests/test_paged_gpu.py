"""GPU parity of the paged, variable-length decode against the fp64 oracle.

Every sequence is checked on its own: the oracle decodes the sequence's
contiguous keys and values (before they were scattered into cache blocks)
with one streaming pass at the sequence's own threshold -- factor / L_b, or
the per-sequence value given -- which is what chained splits decide.  Masks
are graded with the margin rule, outputs against the oracle re-run with the
GPU's mask forced (rel-L2 <= 1e-2); mask entries past a sequence's end must
read 2 (not visited).
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.grading import ROW_FACTOR, grade_masks, max_row_rel_l2, rel_l2
from synth import paged_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def log(*a):
    print(*a, flush=True)


def run_paged(ss, x, scale, factor=0.0, thresholds=None, num_splits=0, latent_dv=None):
    B, Hq, D = x["q"].shape
    Hkv = x["k_cache"].shape[1]
    Dv = latent_dv or D
    L = int(x["seq_lens"].max())
    mask = torch.full(ss.mask_shape_decode(B, Hkv, L), 255, dtype=torch.uint8, device="cuda")
    nbytes = ss.ss_attn_decode_workspace_bytes(B, Hq, Hkv, L, D, Dv, num_splits)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    thr_t = None if thresholds is None else torch.tensor(thresholds, dtype=torch.float32,
                                                         device="cuda")
    v_cache = None if x["v_cache"] is None else x["v_cache"].cuda()
    out = ss.ss_attn_decode_paged(
        x["q"].cuda(), x["k_cache"].cuda(), v_cache, x["block_table"].cuda(),
        x["seq_lens"].cuda(), max_seq_len=L, dv=latent_dv, scale=scale, factor=factor,
        thresholds=thr_t, num_splits=num_splits, skip_mask=mask, workspace=ws)
    torch.cuda.synchronize()
    timeouts = int(ws[nbytes - 256:nbytes - 252].view(torch.int32).item())
    return out.float().cpu().numpy(), mask.cpu().numpy(), timeouts


def seq_threshold(factor, thresholds, b, L):
    """The fp32 threshold sequence b is decided with (factor / L rounded once)."""
    if thresholds is not None:
        return float(np.float32(thresholds[b]))
    return float(np.float32(factor / L))


def check_paged(ss, x, scale, name, factor=0.0, thresholds=None, num_splits=0, latent_dv=None):
    out, mask, timeouts = run_paged(ss, x, scale, factor, thresholds, num_splits, latent_dv)
    assert timeouts == 0, f"{name}: {timeouts} look-back waits gave up"
    lens = [int(v) for v in x["seq_lens"]]
    skipped = visited = 0
    for b, L in enumerate(lens):
        thr = seq_threshold(factor, thresholds, b, L)
        qb = x["q"][b:b + 1]
        kb = x["k_seqs"][b][None]
        vb = None if x["v_seqs"] is None else x["v_seqs"][b][None]
        ref = oracle.decode(qb, kb, vb, scale, thr, 1, latent_dv=latent_dv)
        nK = -(-L // 128)
        mb = mask[b:b + 1, :, :nK]
        assert np.isin(mb, (0, 1)).all(), f"{name}: sequence {b} has unwritten mask entries"
        assert (mask[b, :, nK:] == 2).all(), f"{name}: tiles past sequence {b}'s end not 2"
        gr = grade_masks(mb, ref["mask"], ref["delta"], thr, None)
        assert gr["ok"], f"{name}: sequence {b} mask {gr}"
        forced = oracle.decode(qb, kb, vb, scale, thr, 1, latent_dv=latent_dv, force_mask=mb)
        err = rel_l2(out[b:b + 1], forced["out"])
        assert err <= 1e-2, f"{name}: sequence {b} (L={L}, thr={thr:.3g}) rel-L2 {err}"
        row = max_row_rel_l2(out[b:b + 1], forced["out"])
        assert row <= ROW_FACTOR * 1e-2, f"{name}: sequence {b} worst row rel-L2 {row}"
        skipped += int((mb == 1).sum())
        visited += mb.size
    log(f"[paged {name}] lengths={lens} skip={skipped / max(visited, 1):.3f}")


PAGED_CASES = [
    # name, lengths, Hq, Hkv, D, block_size, r, factor, thresholds, num_splits
    ("mixed_bs16", [1, 127, 128, 129, 1000, 5000], 8, 2, 128, 16, 9.0, 50.0, None, 0),
    ("g8_bs128", [3000, 300, 4097], 16, 2, 128, 128, 9.0, 80.0, None, 0),
    ("mha_d64_bs32", [700, 64, 2000], 4, 4, 64, 32, 9.0, 30.0, None, 0),
    ("g2_d64_bs64", [2049, 1], 4, 2, 64, 64, 9.0, 100.0, None, 3),
    ("per_seq_thresholds", [2500, 800, 129, 4000], 8, 2, 128, 64, 9.0, 0.0,
     [0.05, 0.0, 0.5, 1.0], 0),
    ("dense", [1000, 3000], 8, 2, 128, 16, 3.0, 0.0, None, 0),
    ("many_splits", [5000, 100, 2600], 8, 2, 128, 16, 9.0, 40.0, None, 40),
    ("long_chain_g1", [20000, 7000], 2, 2, 128, 128, 9.0, 200.0, None, 0),
    ("gqa5_bs32", [3000, 129, 1700], 10, 2, 128, 32, 9.0, 60.0, None, 0),
    ("mqa16_bs16", [4000, 1000], 16, 1, 128, 16, 9.0, 60.0, None, 0),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_decode(ss, case):
    name, lens, Hq, Hkv, D, bs, r, factor, thresholds, S = case
    x = paged_decode(zlib.crc32(name.encode()) % 10000, lens, Hq, Hkv, D, D, 16, r, bs)
    check_paged(ss, x, 1 / math.sqrt(D), name, factor, thresholds, S)


PAGED_LATENT_CASES = [
    # name, lengths, Hq, block_size, r, factor, thresholds, num_splits (one
    # latent head: D = 576, value = the first 512 columns of the key row)
    ("mla128_bs64_mixed", [3000, 129, 8197], 128, 64, 9.0, 300.0, None, 0),
    ("mla64_bs32_per_seq", [2500, 1, 700], 64, 32, 9.0, 0.0, [0.05, 0.0, 1.0], 0),
    ("mla128_bs128_dense", [1000, 2000], 128, 128, 3.0, 0.0, None, 0),
    ("mla128_long_chain", [20000, 3000], 128, 64, 9.0, 400.0, None, 0),
    ("mla64_splits", [5000, 300, 2600], 64, 32, 9.0, 150.0, None, 7),
]


@pytest.mark.parametrize("case", PAGED_LATENT_CASES, ids=[c[0] for c in PAGED_LATENT_CASES])
def test_paged_latent_decode(ss, case):
    name, lens, Hq, bs, r, factor, thresholds, S = case
    x = paged_decode(zlib.crc32(name.encode()) % 10000, lens, Hq, 1, 576, 512, 16, r, bs,
                     latent=True)
    check_paged(ss, x, 1 / 24, name, factor, thresholds, S, latent_dv=512)


def test_paged_equals_contiguous_decode(ss):
    """Equal lengths and an identity block table: the paged call reads the
    same rows as the contiguous decode with chained splits, so the masks agree
    exactly and the outputs to rounding (the two instantiations may contract
    floating-point operations differently)."""
    from synth import clustered_decode

    B, Hq, Hkv, L, D, bs = 3, 8, 2, 2000, 128, 16
    x = clustered_decode(321, B, Hq, Hkv, L, D, D, 16, 9.0)
    nblk = -(-L // bs)
    k_cache = torch.zeros((B * nblk, Hkv, bs, D), dtype=torch.bfloat16)
    v_cache = torch.zeros_like(k_cache)
    for b in range(B):
        for j in range(nblk):
            r0, r1 = j * bs, min((j + 1) * bs, L)
            k_cache[b * nblk + j, :, : r1 - r0] = x["k"][b, :, r0:r1]
            v_cache[b * nblk + j, :, : r1 - r0] = x["v"][b, :, r0:r1]
    table = torch.arange(B * nblk, dtype=torch.int32).reshape(B, nblk)
    lens = torch.full((B,), L, dtype=torch.int32)
    thr = 0.05
    scale = 1 / math.sqrt(D)
    S = ss.ss_decode_num_splits(B, Hq, Hkv, L, D, D)
    mask_a = torch.empty(ss.mask_shape_decode(B, Hkv, L), dtype=torch.uint8, device="cuda")
    mask_b = torch.empty_like(mask_a)
    a = ss.ss_attn_decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), scale=scale,
                          threshold=thr, num_splits=S, skip_mask=mask_a)
    b = ss.ss_attn_decode_paged(x["q"].cuda(), k_cache.cuda(), v_cache.cuda(), table.cuda(),
                                lens.cuda(), max_seq_len=L, scale=scale,
                                thresholds=torch.full((B,), thr, dtype=torch.float32,
                                                      device="cuda"),
                                num_splits=S, skip_mask=mask_b)
    torch.cuda.synchronize()
    assert torch.equal(mask_a, mask_b)
    assert rel_l2(b.float().cpu().numpy(), a.float().cpu().numpy()) <= 1e-3
