"""Length-normalised thresholds on the GPU decode against a closed form.

The BLASST summary page ("Calibratie en Thresholding") scales the threshold
inversely with the context length, threshold = a / L, and reports that the
resulting sparsity stays put from 4K to 64K+ tokens.  When the scaled scores
are i.i.d. standard Gumbel (``synth.gumbel_decode``) that stability is exact:
the expected skip fraction of one streaming pass is
(1/n) * sum_{j<n} a j / (a j + L) over n = L/128 tiles, which for a fixed
``a`` depends on L only through a 1/n term (derivation next to
``gumbel_expected_skip`` in the oracle pins).

Here the GQA decode kernel (B x Hq32/Hkv8, D128, chained splits with the
automatic split count, the launch the benchmark times) runs at 4K, 32K and
200K keys with ``a`` solved from the closed form for 70 % and 90 % skip at
32K and then kept at every length; its mean per-stream skip must sit within
4 standard errors (+0.01 for bf16 rounding of the stored scores) of the
closed form at that length, and 4 sampled
(batch, KV head) streams are graded tile by tile against the oracle.
"""

import math

import numpy as np
import pytest
import torch

from synth import gumbel_decode
from tests.test_oracle_pins import gumbel_expected_skip
from tests.test_parity_gpu import check_decode, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def factor_for(L, target):
    """The a whose closed-form skip fraction at length L is ``target``."""
    lo, hi = 1e-3, 1e9
    for _ in range(200):
        mid = math.sqrt(lo * hi)
        if gumbel_expected_skip(L, mid) < target:
            lo = mid
        else:
            hi = mid
    return math.sqrt(lo * hi)


@pytest.mark.parametrize("L,B", [(4096, 16), (32768, 16), (204800, 4)])
def test_length_scaled_threshold_matches_closed_form(ss, L, B):
    Hq, Hkv, D = 32, 8, 128
    scale = 1 / math.sqrt(D)
    log(f"[stability] generating B={B} L={L}")
    x = gumbel_decode(6000 + L // 4096, B, Hq, Hkv, L, D, D, scale)
    rng = np.random.default_rng(L)
    pairs = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, Hkv, 4))})
    for target in (0.7, 0.9):
        a = factor_for(32768, target)  # one factor for every length
        thr = a / L
        want = gumbel_expected_skip(L, a)
        _, mask = check_decode(ss, x, scale, thr, 0, pairs=pairs, name=f"gumbel_{L}_{target}")
        per_stream = (mask == 1).mean(axis=2).ravel()
        se = per_stream.std(ddof=1) / math.sqrt(per_stream.size)
        got = float(per_stream.mean())
        log(f"[stability] L={L} a={a:.1f} thr={thr:.4g} skip={got:.4f} closed form={want:.4f} "
            f"se={se:.4f}")
        assert abs(got - want) <= 4 * se + 0.01, (L, target, got, want, se)
