"""Pins of the fp64 backward oracle (gradients of the skip-softmax prefill with
its skip decisions held fixed).

None of these re-derives the oracle's formulas: they compare it with torch's
automatic differentiation of textbook attention (no skipping), with finite
differences of the oracle's *forward* streaming pass replaying the same skip
mask, and with invariants of softmax attention.

Page references: the vLLM-Omni design page "Skip-Softmax" ("The
online-softmax pass") and the BLASST summary page (arXiv 2512.12087,
"Belangrijkste Bijdragen": sparsity-aware training).
"""

import numpy as np
import pytest
import torch

import oracle
from synth import clustered_prefill


def inputs(seed, B=1, Hq=2, Hkv=1, Lq=300, Lk=300, D=16, Dv=8, r=6.0, n_c=6):
    x = clustered_prefill(seed, B, Hq, Hkv, Lq, Lk, D, Dv, n_c, r, query_mode="tile",
                          dtype="f32")
    rng = np.random.default_rng(seed + 77)
    do = rng.standard_normal((B, Hq, Lq, Dv))
    return oracle.to_f64(x["q"]), oracle.to_f64(x["k"]), oracle.to_f64(x["v"]), do


def rel_err(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def torch_attention_grads(q, k, v, do, scale, causal):
    """Textbook attention in fp64 through torch's softmax and autograd; KV
    heads repeated for the query heads that read them; bottom-right causal."""
    Hq, Hkv = q.shape[1], k.shape[1]
    Lq, Lk = q.shape[2], k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if causal:
        hidden = torch.arange(Lk)[None, :] > torch.arange(Lq)[:, None] + (Lk - Lq)
        s = s.masked_fill(hidden, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)  # rows that see no key
    o = torch.matmul(p, vv)
    (o * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(Lq=300, Lk=300), dict(Lq=130, Lk=300), dict(Lq=300, Lk=257),
    dict(Hq=4, Hkv=2, Lq=200, Lk=200), dict(Hq=3, Hkv=1, Lq=129, Lk=129),
])
def test_dense_gradients_match_autograd(causal, shape):
    """No skipped tile: the gradients are those of softmax attention, as torch's
    autograd computes them (1e-10)."""
    q, k, v, do = inputs(5, **shape)
    scale = 0.3
    ref = oracle.prefill_backward(q, k, v, do, scale, causal)
    dq, dk, dv, o = torch_attention_grads(q, k, v, do, scale, causal)
    assert rel_err(ref["out"], o) < 1e-12
    assert rel_err(ref["dq"], dq) < 1e-10
    assert rel_err(ref["dk"], dk) < 1e-10
    assert rel_err(ref["dv"], dv) < 1e-10


@pytest.mark.parametrize("thr", [0.5, 1.0, 3.0])
@pytest.mark.parametrize("causal", [False, True])
def test_skip_gradients_match_finite_differences_of_the_forward(thr, causal):
    """With a real skip mask from the forward, the oracle's gradients equal
    central finite differences of the forward streaming pass that replays that
    mask (loss = sum dO * O), for sampled elements of q, k and v."""
    q, k, v, do = inputs(11, Hq=2, Hkv=1, Lq=200, Lk=260, D=8, Dv=4, r=8.0)
    scale = 0.35
    fwd = oracle.prefill(q, k, v, scale, causal, thr, tq=32, tk=32)
    mask = fwd["mask"]
    assert (mask == oracle.MASK_SKIPPED).any() and (mask == oracle.MASK_COMPUTED).any()
    g = oracle.prefill_backward(q, k, v, do, scale, causal, mask, tq=32, tk=32)
    assert rel_err(g["out"], fwd["out"]) < 1e-12
    finite = np.isfinite(fwd["lse"])
    assert np.allclose(g["lse"][finite], fwd["lse"][finite], rtol=0, atol=1e-12)

    def loss(args):
        o = oracle.prefill(args["q"], args["k"], args["v"], scale, causal, thr, tq=32, tk=32,
                           force_mask=mask)["out"]
        return float((o * do).sum())

    rng = np.random.default_rng(3)
    h = 1e-5
    for name, grad in [("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])]:
        arr = {"q": q, "k": k, "v": v}[name]
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            base = {"q": q, "k": k, "v": v}
            fd = (loss({**base, name: plus}) - loss({**base, name: minus})) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd,
                                                                             grad[idx])


def test_key_gradient_sums_to_zero():
    """Shifting every key of a KV head by the same vector shifts each row's
    scores by a constant, which softmax ignores, so the key gradients of a KV
    head sum to zero (with any fixed mask)."""
    q, k, v, do = inputs(21, Hq=4, Hkv=2, Lq=260, Lk=260, D=16, Dv=8)
    fwd = oracle.prefill(q, k, v, 0.25, True, 0.1, tq=64, tk=64)
    g = oracle.prefill_backward(q, k, v, do, 0.25, True, fwd["mask"], tq=64, tk=64)
    s = g["dk"].sum(axis=2)
    assert np.abs(s).max() <= 1e-12 * np.abs(g["dk"]).max() * g["dk"].shape[2]


def test_value_gradient_sums_to_the_output_gradient():
    """Every row's weights sum to one over its kept keys, so summed over the
    keys of a KV head, dV equals the sum of dO over the rows that kept a key."""
    q, k, v, do = inputs(31, Hq=2, Hkv=1, Lq=250, Lk=250, D=8, Dv=4)
    fwd = oracle.prefill(q, k, v, 0.3, True, 0.3, tq=32, tk=32)
    g = oracle.prefill_backward(q, k, v, do, 0.3, True, fwd["mask"], tq=32, tk=32)
    rows = np.isfinite(g["lse"])  # rows with at least one kept key
    want = np.einsum("bhrd,bhr->bd", do, rows.astype(float))
    assert np.allclose(g["dv"].sum(axis=2)[:, 0], want, rtol=0, atol=1e-10)


def test_gqa_gradients_equal_mha_with_repeated_kv():
    """A KV head's gradients are the sums of those of the query heads that read
    it, as in multi-head attention with the KV head repeated."""
    q, k, v, do = inputs(41, Hq=4, Hkv=2, Lq=200, Lk=200, D=8, Dv=8)
    fwd = oracle.prefill(q, k, v, 0.3, False, 0.1, tq=64, tk=64)
    g = oracle.prefill_backward(q, k, v, do, 0.3, False, fwd["mask"], tq=64, tk=64)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    gm = oracle.prefill_backward(q, kr, vr, do, 0.3, False, fwd["mask"], tq=64, tk=64)
    assert rel_err(g["dq"], gm["dq"]) < 1e-13
    assert rel_err(g["dk"], gm["dk"].reshape(1, 2, 2, 200, 8).sum(axis=2)) < 1e-13
    assert rel_err(g["dv"], gm["dv"].reshape(1, 2, 2, 200, 8).sum(axis=2)) < 1e-13


def test_row_statistic_is_output_dot_output_gradient():
    """D_r = dO_r . O_r, the per-row term of the softmax derivative."""
    q, k, v, do = inputs(51, Lq=160, Lk=160)
    g = oracle.prefill_backward(q, k, v, do, 0.3, True)
    assert np.allclose(g["D"], (g["out"] * do).sum(axis=-1), rtol=0, atol=1e-12)


def test_skipped_tiles_send_no_gradient():
    """A key tile that every query tile skipped (or did not visit) receives no
    key or value gradient."""
    q, k, v, do = inputs(61, Hq=1, Hkv=1, Lq=256, Lk=256, D=8, Dv=4)
    mask = np.zeros((1, 1, 4, 4), np.uint8)
    mask[0, 0, :, 2] = oracle.MASK_SKIPPED
    g = oracle.prefill_backward(q, k, v, do, 0.3, False, mask, tq=64, tk=64)
    assert np.all(g["dk"][0, 0, 128:192] == 0) and np.all(g["dv"][0, 0, 128:192] == 0)
    assert np.abs(g["dk"][0, 0, :128]).max() > 0
