"""The C-ABI library on the CPU: it loads, exports every declared entry point,
computes the operating point exactly, and rejects bad arguments before
launching anything (no GPU is touched by these tests)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import oracle
from oracle import host as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss_attn.h")


@pytest.fixture(scope="module")
def ss():
    import block_sparse_attention_online_amd as m

    if not os.path.exists(m.library_path()):
        from block_sparse_attention_online_amd.build import build

        build()
    m.lib()
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(ss_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["ss_attn_prefill", "ss_attn_prefill_f32", "ss_attn_prefill_ex", "ss_attn_decode",
              "ss_attn_decode_ex", "ss_attn_decode_partial", "ss_attn_decode_combine",
              "ss_attn_decode_paged", "ss_attn_prefill_backward",
              "ss_attn_prefill_backward_workspace_bytes",
              "ss_attn_decode_workspace_bytes", "ss_decode_num_splits", "ss_factor",
              "ss_threshold", "ss_gate_enabled", "ss_resolve_threshold", "ss_last_error",
              "ss_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(ss):
    exported = subprocess.run(["nm", "-D", "--defined-only", ss.library_path()],
                              capture_output=True, text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in exported.splitlines() if ln.strip()}
    for n in declared_functions():
        assert n in syms, n
        assert hasattr(ss.lib(), n)


def test_missing_library_fails_loudly(ss, monkeypatch, tmp_path):
    """Without the built library every entry point raises; there is no
    fallback that would compute anything elsewhere."""
    monkeypatch.setattr(ss, "_LIB", None)
    monkeypatch.setattr(ss, "library_path", lambda: str(tmp_path / "libssattn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ss.lib()
    with pytest.raises(RuntimeError, match="missing"):
        ss.ss_version()


def test_version(ss):
    assert "gfx950" in ss.ss_version()


# --------------------------------------------------------------------------- operating point

@pytest.mark.parametrize("a,b,s,L", [(2.0, 0.0, 0.7, 32768), (1.5, math.log(2), 1.0, 1000),
                                     (0.3, 4.0, 0.9, 32760), (7.0, -1.0, 0.0, 5)])
def test_factor_calibrated_matches_closed_form(ss, a, b, s, L):
    f = ss.ss_factor("calibrated", a=a, b=b, target_sparsity=s, seqlen=L)
    assert f == pytest.approx(H.factor_calibrated(a, b, s), rel=1e-15)
    assert ss.ss_threshold(f, L) == pytest.approx(H.threshold(f, L), rel=1e-15)


def test_factor_direct_and_threshold(ss):
    assert ss.ss_factor("direct", threshold=1e-3, seqlen=32768) == pytest.approx(32.768, rel=1e-15)
    assert ss.ss_threshold(32.768, 32768) == pytest.approx(1e-3, rel=1e-15)
    assert ss.ss_factor("calibrated", a=2.0, b=0.0, target_sparsity=0.5, seqlen=10) == 2.0


@pytest.mark.parametrize("t,D", [(1.0, 0.7), (0.7, 0.7), (0.6, 0.7), (0.2, 0.7), (None, 0.7),
                                 (None, None), (0.95, None), (0.0, 0.0)])
def test_gate_matches_truth_table(ss, t, D):
    assert ss.ss_gate_enabled(t, D) == H.gate_enabled(t, D)


def test_resolve_threshold(ss):
    # gate off -> dense
    assert ss.ss_resolve_threshold("direct", threshold=0.01, seqlen=100, timestep=1.0,
                                   disabled_until=0.7) == 0.0
    # direct: the user threshold unchanged (no factor round trip)
    assert ss.ss_resolve_threshold("direct", threshold=0.0123, seqlen=32760, timestep=0.6,
                                   disabled_until=0.7) == pytest.approx(0.0123, rel=1e-7)
    # calibrated: a*exp(b*s)/L
    got = ss.ss_resolve_threshold("calibrated", a=3.0, b=2.0, target_sparsity=0.7, seqlen=32760,
                                  timestep=0.2, disabled_until=0.7)
    assert got == pytest.approx(3.0 * math.exp(1.4) / 32760, rel=1e-7)
    # no timestep published while gating is configured -> dense
    assert ss.ss_resolve_threshold("calibrated", a=3.0, b=2.0, target_sparsity=0.7, seqlen=10,
                                   disabled_until=0.7) == 0.0


def test_calibrated_threshold_is_clamped_to_one(ss):
    """Above 1 the test no longer bounds a skipped key's weight: a fitted
    factor that asks for more is clamped and reported as not reachable."""
    from block_sparse_attention_online_amd.calibrate import calibrated_threshold

    thr, ok = calibrated_threshold(3.0, 2.0, 0.7, 32760)
    assert ok and thr == pytest.approx(3.0 * math.exp(1.4) / 32760, rel=1e-7)
    thr, ok = calibrated_threshold(3.0, 2.0, 0.7, 20)        # 3 e^1.4 / 20 = 0.608
    assert ok and thr == pytest.approx(3.0 * math.exp(1.4) / 20, rel=1e-7)
    thr, ok = calibrated_threshold(3.0, 2.0, 0.7, 12)        # 1.014 asked for
    assert (thr, ok) == (1.0, False)
    thr, ok = calibrated_threshold(5e5, 1.0, 0.9, 32760)
    assert (thr, ok) == (1.0, False)
    # gated off: dense, whatever the fit
    assert calibrated_threshold(5e5, 1.0, 0.9, 32760, timestep=1.0, disabled_until=0.7) == (0.0, True)


@pytest.mark.parametrize("kw", [dict(mode="calibrated", a=1.0, b=1.0, target_sparsity=1.5),
                                dict(mode="calibrated", a=float("nan"), b=1.0),
                                dict(mode="calibrated", a=-1.0, b=0.0),
                                dict(mode="direct", threshold=-1.0),
                                dict(mode="direct", threshold=float("inf")),
                                dict(mode="direct", threshold=0.1, seqlen=0),
                                dict(mode=7)])
def test_factor_rejects_bad_domain(ss, kw):
    kw.setdefault("seqlen", 100)
    mode = kw.pop("mode")
    with pytest.raises(ss.SSError) as e:
        ss.ss_factor(mode, **kw)
    assert e.value.code == -1
    assert ss.ss_last_error()


def test_threshold_rejects_bad_domain(ss):
    for f, L in [(1.0, 0), (-1.0, 10), (float("nan"), 10)]:
        with pytest.raises(ss.SSError):
            ss.ss_threshold(f, L)


# --------------------------------------------------------------------------- split policy

def test_split_policy_is_deterministic_and_bounded(ss):
    # GQA decode, Llama-3.1-8B attention shape at 32K: 128 (batch, kv head)
    # units x 256 tiles, ~2816 workgroups wanted -> 12 tiles per split
    # (within the chained capacity of 16 for a group of 4), 22 splits
    assert ss.ss_decode_num_splits(16, 32, 8, 32768, 128, 128) == 22
    # at 200K keys the chained capacity binds: 16 tiles per split
    assert ss.ss_decode_num_splits(16, 32, 8, 204800, 128, 128) == 100
    # small problems: one tile per split
    assert ss.ss_decode_num_splits(1, 4, 2, 1000, 128, 128) == 8
    # group of 1: capacity 64 tiles
    assert ss.ss_decode_num_splits(64, 64, 64, 65536, 128, 128) == 8
    for L in [1, 100, 128, 129, 1000, 4096, 65536]:
        nK = -(-L // 128)
        s = ss.ss_decode_num_splits(1, 4, 4, L, 128, 128)
        assert 1 <= s <= nK
    assert ss.ss_decode_num_splits(1, 3, 2, 100, 128, 128) == 0  # Hq % Hkv
    # latent decode (576-wide rows, 512 value columns, one latent head): a
    # sub-split runs as one workgroup for all query heads, 256 workgroups
    # wanted, at most 64 tiles per sub-split
    assert ss.ss_decode_num_splits(8, 128, 1, 16384, 576, 512) == 32   # 4 tiles each
    assert ss.ss_decode_num_splits(8, 128, 1, 131072, 576, 512) == 32  # 32 tiles each
    assert ss.ss_decode_num_splits(1, 128, 1, 1 << 20, 576, 512) == 256  # 32 tiles each
    assert ss.ss_decode_num_splits(1, 128, 1, 1 << 23, 576, 512) == 1024  # capped at 64 tiles
    assert ss.ss_decode_num_splits(2, 64, 1, 8192, 576, 512) == 64     # 1 tile each


def test_workspace_bytes(ss):
    # hand layout for B2 Hq8 Hkv2 Lk1000 D=Dv=64, 3 requested splits: 8 tiles;
    # chained -> 3 sub-splits of 3 tiles; independent -> 3 user splits of 3
    # tiles, each within capacity (16 tiles for a group of 4) -> 3 sub-splits
    S = 3
    o = S * 2 * 8 * 64 * 4          # 12288: split outputs
    lse = S * 2 * 8 * 4             # 192 -> 256: split lse
    slots = S * 2 * 2 * 4 * 8       # 384 -> 512: published per-row maxima (64-bit)
    want = o + 256 + 512 + 256      # + the look-back timeout counter block
    assert ss.ss_attn_decode_workspace_bytes(2, 8, 2, 1000, 64, 64, 3) == want
    # long independent splits are cut into chains: 1 split of 40 tiles for a
    # group of 4 (capacity 16) -> 3 sub-splits of 14 tiles
    n = ss.ss_attn_decode_workspace_bytes(1, 4, 1, 5000, 128, 128, 1)
    assert n >= 3 * 4 * 128 * 4
    for args in [(16, 32, 8, 32768, 128, 128, 0), (2, 8, 2, 1000, 64, 64, 99)]:
        assert ss.ss_attn_decode_workspace_bytes(*args) > 0
    # latent decode: split outputs, lse, per-row maxima, the timeout block,
    # then the share-out of a thresholded decode: kept-tile masks (8 B per
    # sub-split), 64 tile indices and a count per sub-split, each head's max
    S = 32  # B8 Hq128 Lk16384: 32 sub-splits of 4 tiles
    o = S * 8 * 128 * 512 * 4
    lse = S * 8 * 128 * 4
    slots = S * 8 * 128 * 8
    share = 2048 + S * 8 * 64 * 4 + 1024 + 8 * 128 * 4
    assert ss.ss_attn_decode_workspace_bytes(8, 128, 1, 16384, 576, 512, 0) == (
        o + lse + slots + 256 + share)


# --------------------------------------------------------------------------- argument checks

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def prefill_call(ss, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, Hq=4, Hkv=2, Lq=256, Lk=256, D=128, Dv=128,
             scale=0.1, causal=1, thr=0.01, mask=None)
    a.update(over)
    return ss.lib().ss_attn_prefill(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                    a["Lq"], a["Lk"], a["D"], a["Dv"], a["scale"], a["causal"],
                                    a["thr"], a["mask"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(B=0), -1), (dict(Lq=-5), -1),
    (dict(Hq=3), -1), (dict(scale=0.0), -1), (dict(scale=float("inf")), -1),
    (dict(thr=-0.1), -1), (dict(thr=float("nan")), -1), (dict(thr=float("inf")), -1),
    (dict(D=96, Dv=96), -2), (dict(D=128, Dv=64), -2), (dict(Lk=(1 << 24) + 1), -1),
])
def test_prefill_rejects_before_launch(ss, over, code):
    assert prefill_call(ss, **over) == code
    assert ss.ss_last_error()


def test_prefill_ex_rejects_unknown_order_and_dtype(ss):
    p = ss._PrefillParams(0x1000, 0x1000, 0x1000, 0x1000, 1, 1, 1, 128, 128, 128, 128, 0.1, 0.0,
                          0, 0, 5, None)
    assert ss.lib().ss_attn_prefill_ex(ctypes.byref(p), None) == -1
    p.order, p.dtype = 0, 9
    assert ss.lib().ss_attn_prefill_ex(ctypes.byref(p), None) == -1
    assert ss.lib().ss_attn_prefill_ex(None, None) == -1


def test_prefill_rejects_bad_granularity(ss):
    p = ss._PrefillParams(0x1000, 0x1000, 0x1000, 0x1000, 1, 1, 1, 128, 128, 128, 128, 0.1, 0.0,
                          0, 0, 0, None, 7, None)
    assert ss.lib().ss_attn_prefill_ex(ctypes.byref(p), None) == -1
    assert "granularity" in ss.ss_last_error()
    p.granularity, p.row_mask_out = 0, 0x1000  # a row mask needs per-row decisions
    assert ss.lib().ss_attn_prefill_ex(ctypes.byref(p), None) == -1
    assert "row_mask_out" in ss.ss_last_error()


def test_backward_workspace_bytes(ss):
    # per (batch, head, 128-row query tile): 128 lse values and 128 row dots, fp32
    assert ss.ss_attn_prefill_backward_workspace_bytes(1, 32, 16384) == 32 * 128 * 1024
    assert ss.ss_attn_prefill_backward_workspace_bytes(2, 3, 129) == 2 * 3 * 2 * 1024
    assert ss.ss_attn_prefill_backward_workspace_bytes(1, 1, 1) == 1024
    for bad in [(0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, (1 << 24) + 1)]:
        assert ss.ss_attn_prefill_backward_workspace_bytes(*bad) == 0


def backward_call(ss, **over):
    a = dict(q=0x1000, k=0x1000, v=0x1000, out=0x1000, dout=0x1000, lse=0x1000, skip_mask=None,
             dq=0x1000, dk=0x1000, dv=0x1000, B=1, Hq=4, Hkv=2, Lq=256, Lk=256, D=128, Dv=128,
             scale=0.1, causal=1, dtype=0, workspace=0x1000, workspace_bytes=1 << 30)
    a.update(over)
    p = ss._PrefillBwdParams(*[a[f] for f, _ in ss._PrefillBwdParams._fields_])
    return ss.lib().ss_attn_prefill_backward(ctypes.byref(p), None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(dout=None), -1), (dict(lse=None), -1), (dict(dk=None), -1),
    (dict(B=0), -1), (dict(Lk=-1), -1), (dict(Hq=3), -1), (dict(scale=0.0), -1),
    (dict(scale=float("nan")), -1), (dict(Lq=(1 << 24) + 1), -1), (dict(dtype=7), -1),
    (dict(dtype=1), -2), (dict(D=96, Dv=96), -2), (dict(D=128, Dv=64), -2),
    (dict(workspace=None), -4), (dict(workspace_bytes=4 * 2 * 1024 - 1), -4),
])
def test_backward_rejects_before_launch(ss, over, code):
    assert backward_call(ss, **over) == code
    assert ss.ss_last_error()
    assert ss.lib().ss_attn_prefill_backward(None, None) == -1


def test_struct_layouts_match_header(ss, tmp_path):
    """Every field of the parameter structs sits at the offset the C compiler
    gives it in include/ss_attn.h (the binding fills them by position)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs gcc and the HIP headers")
    structs = {"ss_prefill_params": ss._PrefillParams, "ss_decode_params": ss._DecodeParams,
               "ss_decode_paged_params": ss._DecodePagedParams,
               "ss_prefill_bwd_params": ss._PrefillBwdParams}
    lines = ['#include "ss_attn.h"', "#include <stdio.h>", "#include <stddef.h>",
             "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True,
                               text=True).stdout.splitlines():
        name, field, val = line.split()
        got[(name, field)] = int(val)
    for name, cls in structs.items():
        assert got[(name, "sizeof")] == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)


def decode_call(ss, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, Lk=1000, D=128, Dv=128,
             scale=0.1, thr=0.01, S=0, mask=None, ws=FAKE, wsb=1 << 30, mode=0, gran=0,
             rmask=None)
    a.update(over)
    if a["mode"] != 0 or a["gran"] != 0 or a["rmask"] is not None:
        p = ss._DecodeParams(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"], a["Lk"],
                             a["D"], a["Dv"], a["scale"], a["thr"], a["S"], a["mode"], a["mask"],
                             a["ws"], a["wsb"], a["gran"], a["rmask"])
        return ss.lib().ss_attn_decode_ex(ctypes.byref(p), None)
    return ss.lib().ss_attn_decode(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"],
                                   a["Lk"], a["D"], a["Dv"], a["scale"], a["thr"], a["S"],
                                   a["mask"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(Lk=0), -1), (dict(Hq=7), -1),
    (dict(S=-1), -1), (dict(thr=-1.0), -1), (dict(scale=-0.5), -1),
    (dict(v=None, Dv=256), -1),                     # latent value wider than the key row
    (dict(Hq=48, Hkv=2), -2),                       # group of 24 heads
    (dict(D=96, Dv=96), -2), (dict(v=None, Dv=64), -2),
    (dict(ws=None), -4), (dict(wsb=100), -4), (dict(mode=7), -1),
    (dict(gran=2), -1), (dict(rmask=FAKE), -1),    # row mask without per-row decisions
    (dict(v=None, D=576, Dv=512, Hq=128, Hkv=1, gran=1), -2),  # per-row latent decode
])
def test_decode_rejects_before_launch(ss, over, code):
    assert decode_call(ss, **over) == code
    assert ss.ss_last_error()


def test_binding_refuses_cpu_tensors(ss):
    import torch

    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ss.ss_attn_prefill(q, q, q)
    with pytest.raises(ValueError, match="GPU tensor"):
        ss.ss_attn_decode(q[:, :, 0], q, q)


def paged_call(ss, **over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, thr=None, out=FAKE, B=2, Hq=8, Hkv=2,
             D=128, Dv=128, bs=16, mb=100, nb=300, L=1600, scale=0.1, factor=10.0, S=0,
             mask=None, ws=FAKE, wsb=1 << 30)
    a.update(over)
    p = ss._DecodePagedParams(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["thr"], a["out"],
                              a["B"], a["Hq"], a["Hkv"], a["D"], a["Dv"], a["bs"], a["mb"],
                              a["nb"], a["L"], a["scale"], a["factor"], a["S"], a["mask"],
                              a["ws"], a["wsb"])
    return ss.lib().ss_attn_decode_paged(ctypes.byref(p), None)


@pytest.mark.parametrize("over,code", [
    (dict(bt=None), -1), (dict(sl=None), -1), (dict(B=0), -1), (dict(nb=0), -1),
    (dict(bs=24), -1), (dict(bs=256), -1), (dict(bs=8), -1),
    (dict(L=1601), -1),                              # more keys than 100 blocks of 16
    (dict(factor=-1.0), -1), (dict(factor=float("nan")), -1), (dict(scale=0.0), -1),
    (dict(Hq=9), -1), (dict(D=96, Dv=96), -2), (dict(Hq=48, Hkv=2), -2),
    (dict(ws=None), -4), (dict(wsb=64), -4),
    # a latent cache (v_cache NULL): only D 576 / Dv 512 with 64 or 128 heads,
    # blocks of 32 keys or more
    (dict(vc=None), -2),
    (dict(vc=None, Hq=128, Hkv=1, D=576, Dv=512, bs=16, mb=200), -2),
    (dict(vc=None, Hq=96, Hkv=1, D=576, Dv=512, bs=64, mb=50), -2),
    (dict(vc=None, Hq=128, Hkv=1, D=576, Dv=512, bs=64, mb=50, wsb=64), -4),
])
def test_paged_decode_rejects_before_launch(ss, over, code):
    assert paged_call(ss, **over) == code
    assert ss.ss_last_error()



def noalloc_call(ss, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, Lk=1000, D=128, Dv=128,
             scale=0.1, thr=0.01, S=0, mask=None)
    a.update(over)
    return ss.lib().ss_attn_decode_noalloc(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"],
                                           a["Hkv"], a["Lk"], a["D"], a["Dv"], a["scale"],
                                           a["thr"], a["S"], a["mask"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(Lk=0), -1), (dict(Hq=7), -1),
    (dict(S=-1), -1), (dict(thr=-1.0), -1), (dict(scale=float("nan")), -1),
    (dict(Hq=48, Hkv=2), -2), (dict(D=96, Dv=96), -2),
    # an explicit split count whose workspace (2^15 splits x 16 x 32 rows x 129
    # floats ~ 8.7 GB) exceeds the fixed array
    (dict(B=16, Hq=32, Hkv=8, Lk=1 << 22, S=1 << 15), -4),
])
def test_noalloc_decode_rejects_before_touching_a_device(ss, over, code):
    assert noalloc_call(ss, **over) == code
    msg = ss.ss_last_error()
    assert msg
    if code == -4:
        assert "allocation-free" in msg and str(ss.DECODE_NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_scratch_size_matches_header(ss):
    src = open(HEADER).read()
    m = re.search(r"#define SS_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ss.DECODE_NOALLOC_SCRATCH_BYTES


def test_noalloc_fits_the_measured_decode_workloads(ss):
    # GQA decode, Llama-3.1-8B shape at 32K keys: the automatic split count fits
    assert ss.ss_attn_decode_workspace_bytes(16, 32, 8, 32768, 128, 128, 0) <= \
        ss.DECODE_NOALLOC_SCRATCH_BYTES
    # latent decode, 8 sequences x 128 heads: the automatic count needs more,
    # a lower count fits (the entry point lowers it by itself)
    assert ss.ss_attn_decode_workspace_bytes(8, 128, 1, 131072, 576, 512, 0) > \
        ss.DECODE_NOALLOC_SCRATCH_BYTES
    assert ss.ss_attn_decode_workspace_bytes(8, 128, 1, 131072, 576, 512, 16) <= \
        ss.DECODE_NOALLOC_SCRATCH_BYTES


def test_lookback_query_rejects_bad_arguments(ss):
    p = ss._DecodeParams(FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 1000, 128, 128, 0.1, 0.01, 0, 0, None,
                         FAKE, 1 << 30, 0, None)
    assert ss.lib().ss_attn_decode_lookback_timeouts(ctypes.byref(p), None, 0, None) == -1
    n = ctypes.c_uint()
    p.workspace = None
    assert ss.lib().ss_attn_decode_lookback_timeouts(ctypes.byref(p), ctypes.byref(n), 0,
                                                     None) == -4
    p.workspace, p.Hq = FAKE, 7
    assert ss.lib().ss_attn_decode_lookback_timeouts(ctypes.byref(p), ctypes.byref(n), 0,
                                                     None) == -1
