"""GPU parity of the skip-aware prefill backward, and of the forward's
log-sum-exp output, against the fp64 oracle, through the C ABI.

The backward replays the forward's decisions: the oracle runs with the skip
mask the GPU forward wrote (``oracle.prefill_backward(..., mask=gpu_mask)``)
on the same bf16-rounded inputs and output gradient.  Gradients are graded by
relative L2 error <= 1e-2 (bf16 inputs, fp32 accumulation, bf16 P and dS
operands and bf16 outputs).  Small cases span several tiles with ragged tails
and run the oracle on everything; the full-size case (causal GQA, 16384
tokens, ~70 % of tile pairs skipped) checks the slices the oracle can finish
exactly -- the last two query tiles with the two key tiles only they see, and
one query tile in the middle -- and an identity of the whole dV.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.grading import rel_l2
from synth import WORKLOADS, clustered_prefill, make_inputs, output_gradient

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def log(*a):
    print(*a, flush=True)


def forward(ss, x, scale, causal, thr, order="ascending"):
    q, k, v = (x[n].cuda() for n in "qkv")
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    mask = torch.full(ss.mask_shape_prefill(B, Hq, Lq, Lk), 255, dtype=torch.uint8, device="cuda")
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    out = ss.ss_attn_prefill_ex(q, k, v, scale=scale, causal=causal, threshold=thr,
                                skip_mask=mask, lse=lse, order=order)
    return q, k, v, out, mask, lse


def backward(ss, fwd, do, scale, causal, use_mask=True):
    q, k, v, out, mask, lse = fwd
    g = ss.ss_attn_prefill_backward(q, k, v, out, do.cuda(), lse, mask if use_mask else None,
                                    scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in g]


def skip_fraction(mask):
    visited = np.isin(mask, (0, 1))
    return float((mask[visited] == 1).mean()) if visited.any() else 0.0


# --------------------------------------------------------------------------- forward lse

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal,Lq,Lk", [(True, 300, 300), (False, 260, 390), (True, 400, 200)])
def test_forward_lse_matches_oracle(ss, dtype, causal, Lq, Lk):
    """lse_out of the forward is ln of each row's kept exponential sum: the
    oracle's value for the GPU's own mask (1e-4 absolute; -inf for rows that
    kept no key)."""
    x = clustered_prefill(71, 1, 4, 2, Lq, Lk, 64, 64, 8, 3.0, query_mode="tile", dtype=dtype)
    scale = 0.125
    for thr in (0.0, 0.3):
        _, _, _, _, mask, lse = forward(ss, x, scale, causal, thr)
        torch.cuda.synchronize()
        mask, lse = mask.cpu().numpy(), lse.cpu().numpy()
        ref = oracle.prefill(x["q"], x["k"], x["v"], scale, causal, thr, force_mask=mask)["lse"]
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.all(lse[~fin] == -np.inf)
        err = np.abs(lse[fin] - ref[fin]).max() if fin.any() else 0.0
        log(f"[lse {dtype}] causal={causal} Lq={Lq} Lk={Lk} thr={thr} max |err|={err:.2e}")
        assert err <= 1e-4


# --------------------------------------------------------------------------- small cases

BWD_CASES = [
    # name, B, Hq, Hkv, Lq, Lk, D, causal
    ("mha_causal_300", 1, 2, 2, 300, 300, 128, True),
    ("gqa4_causal_lq_lt_lk", 1, 8, 2, 260, 390, 128, True),
    ("gqa2_noncausal_d64", 2, 4, 2, 333, 270, 64, False),
    ("group3_causal", 1, 3, 1, 384, 384, 128, True),
    ("lq_gt_lk_causal_d64", 1, 2, 1, 400, 200, 64, True),
    ("one_ragged_tile", 1, 2, 1, 50, 77, 128, False),
    ("gqa4_noncausal_640", 1, 4, 1, 640, 640, 128, False),
]


@pytest.mark.parametrize("thr", [0.0, 0.05, 0.5])
@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_small(ss, case, thr):
    name, B, Hq, Hkv, Lq, Lk, D, causal = case
    x = clustered_prefill(zlib.crc32(name.encode()) % 1000 + 17, B, Hq, Hkv, Lq, Lk, D, D, 8, 3.0,
                          query_mode="tile")
    do = output_gradient(5, B, Hq, Lq, D)
    scale = 1.0 / np.sqrt(D)
    fwd = forward(ss, x, scale, causal, thr)
    dq, dk, dv = backward(ss, fwd, do, scale, causal)
    mask = fwd[4].cpu().numpy()
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], do, scale, causal, mask)
    errs = {n: rel_l2(g, ref[n]) for n, g in (("dq", dq), ("dk", dk), ("dv", dv))}
    log(f"[bwd {name}] thr={thr} skip={skip_fraction(mask):.3f} " +
        " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL, (n, e)
        assert np.isfinite({"dq": dq, "dk": dk, "dv": dv}[n]).all()


def test_backward_without_mask_is_dense(ss):
    """skip_mask = NULL takes every visible tile: the same bits as replaying
    the all-computed mask of a threshold-0 forward, and the oracle's dense
    gradients."""
    x = clustered_prefill(23, 1, 4, 2, 300, 300, 128, 128, 8, 3.0, query_mode="tile")
    do = output_gradient(6, 1, 4, 300, 128)
    scale = 0.09
    fwd = forward(ss, x, scale, True, 0.0)
    assert np.isin(fwd[4].cpu().numpy(), (0, 2)).all()
    with_mask = backward(ss, fwd, do, scale, True, use_mask=True)
    without = backward(ss, fwd, do, scale, True, use_mask=False)
    for a, b in zip(with_mask, without):
        assert np.array_equal(a, b)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], do, scale, True)
    for n, g in zip(("dq", "dk", "dv"), without):
        assert rel_l2(g, ref[n]) <= TOL


def test_backward_skipped_pairs_send_nothing(ss):
    """A key tile that every query tile skipped gets exactly zero dK and dV; a
    query tile that skipped every key tile gets exactly zero dQ.  The mask is
    planted, so the forward's output and lse come from the oracle run with that
    mask (the backward takes them as inputs)."""
    x = clustered_prefill(29, 1, 2, 1, 512, 512, 128, 128, 8, 3.0, query_mode="tile")
    do = output_gradient(7, 1, 2, 512, 128)
    scale = 0.09
    mask = np.zeros((1, 2, 4, 4), np.uint8)
    mask[:, :, :, 2] = 1   # key tile 2 skipped by everyone
    mask[:, 1, 3, :] = 1   # head 1, query tile 3 skipped everything
    fo = oracle.prefill(x["q"], x["k"], x["v"], scale, False, 0.0, force_mask=mask)
    q, k, v = (x[n].cuda() for n in "qkv")
    out = torch.from_numpy(fo["out"]).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(fo["lse"]).float().cuda()
    g = ss.ss_attn_prefill_backward(q, k, v, out, do.cuda(), lse, torch.from_numpy(mask).cuda(),
                                    scale=scale, causal=False)
    torch.cuda.synchronize()
    dq, dk, dv = [t.float().cpu().numpy() for t in g]
    assert np.all(dk[0, 0, 256:384] == 0) and np.all(dv[0, 0, 256:384] == 0)
    assert np.all(dq[0, 1, 384:512] == 0)
    assert np.abs(dk[0, 0, :256]).max() > 0 and np.abs(dq[0, 0, 384:]).max() > 0
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], do, scale, False, mask)
    for n, g in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        assert rel_l2(g, ref[n]) <= TOL, n


def test_backward_is_deterministic(ss):
    x = clustered_prefill(31, 1, 8, 2, 700, 700, 128, 128, 8, 3.0, query_mode="tile")
    do = output_gradient(8, 1, 8, 700, 128)
    fwd = forward(ss, x, 0.09, True, 0.3)
    a = backward(ss, fwd, do, 0.09, True)
    b = backward(ss, fwd, do, 0.09, True)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


# --------------------------------------------------------------------------- full size

def test_backward_gqa_16k_full_size_sampled(ss):
    """Causal GQA prefill at full size (B1 Hq32 Hkv8 L16384 D128) at a
    threshold that skips ~70 % of the visited tile pairs (threshold 1 with the
    diagonal tile first: ~68 %), backward over the whole call.  The oracle
    checks (KV heads 0 and 5, all four query heads of each): the last two
    query tiles with the two key tiles only they see, and query tile 61 (keys
    up to its diagonal); the dV of every KV head must sum over keys to the sum
    of dO over the rows of its query heads."""
    w = WORKLOADS["gqa_prefill_16k"]
    x = make_inputs(w)
    L, g = w.Lq, w.Hq // w.Hkv
    do = output_gradient(9, 1, w.Hq, L, w.Dv)
    fwd = forward(ss, x, w.scale, True, 1.0, order="diag_first")
    dq, dk, dv = backward(ss, fwd, do, w.scale, True)
    mask = fwd[4].cpu().numpy()
    lse = fwd[5].cpu().numpy()
    s = skip_fraction(mask)
    log(f"[bwd gqa16k] skip={s:.3f}")
    assert 0.5 <= s <= 0.9
    nQ = L // 128
    for hk in (0, 5):
        heads = list(range(hk * g, (hk + 1) * g))
        # last two query tiles; key tiles nQ-2, nQ-1 are seen only by them
        r0 = L - 256
        ref = oracle.prefill_backward(x["q"][:, heads, r0:], x["k"][:, [hk]], x["v"][:, [hk]],
                                      do[:, heads, r0:], w.scale, True, mask[:, heads, nQ - 2:])
        e = {"dq": rel_l2(dq[:, heads, r0:], ref["dq"]),
             "dk": rel_l2(dk[:, [hk], r0:], ref["dk"][:, :, r0:]),
             "dv": rel_l2(dv[:, [hk], r0:], ref["dv"][:, :, r0:])}
        # query tile 61 with the keys up to its diagonal
        i = 61
        rows = slice(i * 128, (i + 1) * 128)
        refm = oracle.prefill_backward(x["q"][:, heads, rows], x["k"][:, [hk], :(i + 1) * 128],
                                       x["v"][:, [hk], :(i + 1) * 128], do[:, heads, rows],
                                       w.scale, True, mask[:, heads, i:i + 1, :i + 1])
        e["dq61"] = rel_l2(dq[:, heads, rows], refm["dq"])
        log(f"[bwd gqa16k] kv head {hk}: " + " ".join(f"{n}={v:.2e}" for n, v in e.items()))
        for n, v in e.items():
            assert v <= TOL, (hk, n, v)
    # every row keeps its diagonal tile (visited first, so never skipped), so
    # its weights sum to one: sum over keys of dV = sum over the group's rows of dO
    assert np.isfinite(lse).all()
    do_np = do.float().numpy()
    for hk in range(w.Hkv):
        want = do_np[0, hk * g:(hk + 1) * g].astype(np.float64).sum(axis=(0, 1))
        got = dv[0, hk].astype(np.float64).sum(axis=0)
        assert rel_l2(got, want) <= 2e-2, hk
