"""Per-workload measurement runs of the skip-softmax hot path on one GPU.

  python -m block_sparse_attention_online_amd.harness prefill [--out FILE]
      causal GQA prefill (B1, Hq32/Hkv8, L16384, D128): skip targets
      0.1 .. 0.8 found by bisection on the kernel's own mask, both visit
      orders, the literal generator (r = 3) and the wide-gap one (r = 9):
      executed TFLOP/s, speedup over threshold 0, error against threshold 0.
  python -m block_sparse_attention_online_amd.harness video [--out FILE]
      video-DiT self-attention (B1, H24, 13x42x60 tokens, D128): the
      calibrated factor a*exp(b*s) fitted on replicate 1 and evaluated on
      replicate 0 at s = 0.5, 0.7, 0.9; timestep gating t = 1.0, 0.6, 0.2 with
      the dense-until point 0.7.
  python -m block_sparse_attention_online_amd.harness latent [--out FILE]
      latent decode (B8, 128 heads, 576-wide latent rows, value = first 512
      columns) at 16K..128K keys, clustered keys (r = 3, r = 9) and keys with
      i.i.d. Gumbel scores: one factor a*exp(0.7 b) fitted so ~70 % of tiles
      skip at every length (chained splits), and the threshold bisected to
      70 % with independent splits; K bytes per second and MFMA rate.
  python -m block_sparse_attention_online_amd.harness paged [--out FILE]
      paged decode of a serving-like batch (32 sequences of 1K..32K keys,
      Hq32/Hkv8, D128, 16-key cache blocks), and of a latent-cache batch (16
      sequences of 4K..64K keys, 128 heads on one 576-wide latent head,
      64-key blocks): one factor, threshold factor / L_b per sequence,
      bisected so ~70 % of the batch's tiles skip; skip per length bucket,
      bytes per second, speedup over threshold 0.
  python -m block_sparse_attention_online_amd.harness decode [--out FILE]
      GQA decode (B16, Hq32/Hkv8, 32768 keys, D128): skip 0.5 / 0.7 / 0.9
      against threshold 0, chained splits.
  python -m block_sparse_attention_online_amd.harness stability [--out FILE]
      GQA decode (Hq32/Hkv8, D128) from 4K to 200K keys, batch sized to ~1 GB
      of K: a threshold bisected at 32K for 70 % / 90 % skip, then used either
      unchanged at every length or as a factor (threshold = factor / L); skip
      and speedup per length for clustered keys (r = 3, r = 9) and for keys
      with i.i.d. Gumbel scores, whose factor / L skip has a closed form.

The method and its parameters: vLLM-Omni design page "Skip-Softmax",
sections "The threshold" and "Timestep gating"; BLASST summary page, section
"Calibratie en Thresholding" (threshold = a / L with a fitted so the
sparsity stays fixed across context lengths).

Every timed call is preceded by a read of a 1 GiB buffer, so no call finds
its K/V in L2 or in the 256 MB last-level cache (a read, not a rewrite: a
rewrite leaves dirty lines whose write-back would land in the timed call);
times are the median of the per-call HIP event times on the current stream.
Calibrated thresholds are clamped to 1 (calibrate.calibrated_threshold); a
target that needs more is reported with reachable = false.  Each run prints one
JSON object per measured point; --out also writes a markdown table.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

from . import (lib, mask_shape_decode, mask_shape_prefill, ss_attn_decode_partial,
               ss_attn_decode_combine, ss_attn_decode_workspace_bytes, ss_attn_prefill_ex,
               ss_decode_num_splits, ss_resolve_threshold)
from .calibrate import bisect_threshold, calibrated_threshold, fit_factor, skip_fraction

BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Median per-call time in ms, with L2 and the last-level cache evicted
    before every call by reading a 1 GiB buffer (a rewrite would leave dirty
    lines whose write-back lands in the timed call)."""

    def __init__(self, flush_bytes: int = 1 << 30):
        self.flush = torch.ones(flush_bytes, dtype=torch.uint8, device="cuda")

    def ms(self, fn, iters: int = 15, warmup: int = 3) -> float:
        for _ in range(warmup):
            fn()
        ts = []
        for i in range(iters):
            self.flush.max()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))


def rel_l2_gpu(a: torch.Tensor, b: torch.Tensor) -> float:
    a, b = a.float(), b.float()
    return float(torch.linalg.norm(a - b) / torch.linalg.norm(b))


def md_table(rows, cols) -> str:
    out = ["| " + " | ".join(cols) + " |", "|" + "---|" * len(cols)]
    for r in rows:
        out.append("| " + " | ".join("" if r.get(c) is None else str(r[c]) for c in cols) + " |")
    return "\n".join(out)


def emit(rec, rows):
    print(json.dumps(rec), flush=True)
    rows.append(rec)


# --------------------------------------------------------------------------- prefill

def prefill_flops(mask_np, D, Dv):
    """Executed MFMA flops: Q.K^T of every visited (query tile, key tile),
    P.V of the kept ones, full 128 x 128 tiles as issued."""
    visited = int((mask_np != 2).sum())
    kept = int((mask_np == 0).sum())
    return 2 * 128 * 128 * D * visited + 2 * 128 * 128 * Dv * kept


def run_prefill_sweep(args):
    from synth import WORKLOADS, make_inputs

    timer, rows = Timer(), []
    targets = [0.1 * i for i in range(1, 9)]
    for r in (3.0, 9.0):
        w = WORKLOADS["gqa_prefill_16k"].replace(r=r)
        x = make_inputs(w)
        q, k, v = (x[n].cuda() for n in "qkv")
        del x
        out = torch.empty_like(q)
        mask = torch.empty(mask_shape_prefill(w.B, w.Hq, w.Lq, w.Lk), dtype=torch.uint8,
                           device="cuda")
        fa = 4.0 * w.B * w.Hq * w.Lq * w.Lk * w.D * 0.5
        for order in ("ascending", "diag_first"):
            def run(thr):
                ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=True, threshold=thr,
                                   skip_mask=mask, order=order)

            def skip_at(thr):
                run(thr)
                torch.cuda.synchronize()
                return skip_fraction(mask)

            dense_ms = timer.ms(lambda: run(0.0))
            dense_out = out.clone()
            dense_fl = prefill_flops(mask.cpu().numpy(), w.D, w.Dv)
            emit({"workload": "gqa_prefill_16k", "r": r, "order": order, "target": 0.0,
                  "threshold": 0.0, "skip": 0.0, "ms": round(dense_ms, 4),
                  "tflops_executed": round(dense_fl / dense_ms / 1e9, 1),
                  "frac_bf16_peak": round(dense_fl / dense_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                  "fa_tflops": round(fa / dense_ms / 1e9, 1), "speedup": 1.0,
                  "rel_l2_vs_dense": 0.0}, rows)
            for tgt in targets:
                thr, s, reach = bisect_threshold(skip_at, tgt, iters=24, tol=0.005)
                ms = timer.ms(lambda: run(thr))
                fl = prefill_flops(mask.cpu().numpy(), w.D, w.Dv)
                emit({"workload": "gqa_prefill_16k", "r": r, "order": order,
                      "target": round(tgt, 2), "threshold": float(f"{thr:.6g}"),
                      "reachable": reach, "skip": round(skip_fraction(mask), 4),
                      "ms": round(ms, 4), "tflops_executed": round(fl / ms / 1e9, 1),
                      "frac_bf16_peak": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                      "fa_tflops": round(fa / ms / 1e9, 1),
                      "speedup": round(dense_ms / ms, 3),
                      "rel_l2_vs_dense": float(f"{rel_l2_gpu(out, dense_out):.3e}")}, rows)
        del q, k, v, out
    cols = ["r", "order", "target", "threshold", "reachable", "skip", "ms", "tflops_executed",
            "frac_bf16_peak", "fa_tflops", "speedup", "rel_l2_vs_dense"]
    return rows, cols


# --------------------------------------------------------------------------- video

def run_video(args):
    from synth import WORKLOADS, make_inputs

    timer, rows = Timer(), []
    w = WORKLOADS["video_dit_32760"]
    L = w.Lk
    fa = 4.0 * w.B * w.Hq * w.Lq * w.Lk * w.D
    grid = [float(f"{t:.3g}") for t in np.logspace(-6, 0, 13)]

    def load(seed):
        t = time.time()
        x = make_inputs(w.replace(seed=seed))
        log(f"[video] generated seed {seed} in {time.time() - t:.1f}s")
        return tuple(x[n].cuda() for n in "qkv")

    out = mask = None
    fits = {}
    # 1. calibration sweep on replicate 1
    q, k, v = load(w.seed + 1)
    out = torch.empty_like(q)
    mask = torch.empty(mask_shape_prefill(w.B, w.Hq, w.Lq, w.Lk), dtype=torch.uint8,
                       device="cuda")
    for order in ("ascending", "diag_first"):
        pts = []
        for thr in grid:
            ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=False, threshold=thr,
                               skip_mask=mask, order=order)
            torch.cuda.synchronize()
            s = skip_fraction(mask)
            emit({"workload": w.name, "replicate": 1, "stage": "sweep", "order": order,
                  "threshold": thr, "skip": round(s, 4)}, rows)
            if 0.02 < s < 0.98:
                pts.append((thr, L, s))
        a, b = fit_factor(pts) if len(pts) >= 2 else (float("nan"), float("nan"))
        fits[order] = (a, b)
        emit({"workload": w.name, "replicate": 1, "stage": "fit", "order": order,
              "a": float(f"{a:.6g}"), "b": float(f"{b:.6g}"), "points": len(pts)}, rows)
    del q, k, v
    # 2. evaluation on replicate 0
    q, k, v = load(w.seed)
    for order in ("ascending", "diag_first"):
        a, b = fits[order]

        def run(thr):
            ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=False, threshold=thr,
                               skip_mask=mask, order=order)

        dense_ms = timer.ms(lambda: run(0.0), iters=9)
        dense_out = out.clone()
        emit({"workload": w.name, "replicate": 0, "stage": "dense", "order": order,
              "ms": round(dense_ms, 3), "fa_tflops": round(fa / dense_ms / 1e9, 1)}, rows)
        if not math.isfinite(a):
            continue
        for tgt in (0.5, 0.7, 0.9):
            thr, reach = calibrated_threshold(a, b, tgt, L)
            ms = timer.ms(lambda: run(thr), iters=9)
            fl = prefill_flops(mask.cpu().numpy(), w.D, w.Dv)
            emit({"workload": w.name, "replicate": 0, "stage": "calibrated", "order": order,
                  "target": tgt, "threshold": float(f"{thr:.6g}"), "reachable": reach,
                  "skip": round(skip_fraction(mask), 4), "ms": round(ms, 3),
                  "tflops_executed": round(fl / ms / 1e9, 1),
                  "frac_bf16_peak": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                  "speedup": round(dense_ms / ms, 3),
                  "rel_l2_vs_dense": float(f"{rel_l2_gpu(out, dense_out):.3e}")}, rows)
        for t in (1.0, 0.6, 0.2):
            thr, reach = calibrated_threshold(a, b, 0.7, L, timestep=t, disabled_until=0.7)
            ms = timer.ms(lambda: run(thr), iters=9)
            emit({"workload": w.name, "replicate": 0, "stage": "gating", "order": order,
                  "timestep": t, "disabled_until": 0.7, "mode": "dense" if thr == 0 else "sparse",
                  "threshold": float(f"{thr:.6g}"), "reachable": reach,
                  "skip": round(skip_fraction(mask), 4), "ms": round(ms, 3)}, rows)
    cols = ["replicate", "stage", "order", "threshold", "reachable", "a", "b", "target",
            "timestep", "mode",
            "skip", "ms", "tflops_executed", "frac_bf16_peak", "fa_tflops", "speedup",
            "rel_l2_vs_dense"]
    return rows, cols


# --------------------------------------------------------------------------- latent decode

def run_latent(args):
    """Latent decode, 16K-128K keys, three key distributions (the clustered
    generator at r = 3 and r = 9, and Gumbel scores): per length the
    threshold bisected to 70 % skip with chained splits, the one factor a
    (b from the sweep) that the method fits for all lengths, and the
    threshold bisected to 70 % with independent splits (each split one
    streaming pass), each timed against threshold 0."""
    from synth import WORKLOADS, gumbel_decode, make_inputs

    timer, rows = Timer(), []
    ctxs = [16, 32, 64, 128]
    grid = [float(f"{t:.3g}") for t in np.logspace(-5, 0, 11)]

    def clustered(r):
        return lambda n: (WORKLOADS[f"mla_decode_{n}k"].replace(r=r),
                          make_inputs(WORKLOADS[f"mla_decode_{n}k"].replace(r=r)))

    def gumbel(n):
        w = WORKLOADS[f"mla_decode_{n}k"]
        return w, gumbel_decode(5100 + n, w.B, w.Hq, 1, w.Lk, 576, 512, w.scale, latent=True)

    for keys, gen in (("clustered r=3", clustered(3.0)), ("clustered r=9", clustered(9.0)),
                      ("gumbel", gumbel)):
        data, pts, per_ctx = {}, [], {}
        for n in ctxs:
            w, x = gen(n)
            q, k = x["q"].cuda(), x["k"].cuda()
            del x
            ws = torch.empty(ss_attn_decode_workspace_bytes(w.B, w.Hq, 1, w.Lk, 576, 512, 0),
                             dtype=torch.uint8, device="cuda")
            mask = torch.empty(mask_shape_decode(w.B, 1, w.Lk), dtype=torch.uint8, device="cuda")
            out = torch.empty((w.B, w.Hq, 512), dtype=torch.bfloat16, device="cuda")

            def part(thr, mode, q=q, k=k, ws=ws, mask=mask, w=w):
                ss_attn_decode_partial(q, k, None, dv=512, scale=w.scale, threshold=thr,
                                       skip_mask=mask, workspace=ws, split_mode=mode)

            def call(thr, mode="chained", part=part, q=q, k=k, ws=ws, out=out):
                part(thr, mode)
                ss_attn_decode_combine(q, k, ws, out, dv=512)

            def skip_at(thr, mode="chained", part=part, mask=mask):
                part(thr, mode)
                torch.cuda.synchronize()
                return skip_fraction(mask)

            for thr in grid:
                s = skip_at(thr)
                if 0.02 < s < 0.98:
                    pts.append((thr, w.Lk, s))
            t70, _, reach = bisect_threshold(skip_at, 0.7, iters=24, tol=0.005)
            i70, _, ireach = bisect_threshold(lambda t, f=skip_at: f(t, "independent"), 0.7,
                                              iters=24, tol=0.005)
            per_ctx[n] = (t70, reach, i70, ireach)
            data[n] = (w, call, skip_at, mask, out)
        a_fit, b = fit_factor(pts) if len(pts) >= 2 else (float("nan"), 0.0)
        # one a for all lengths: ln a = mean over lengths of ln(t70 * L) - 0.7 b
        la = [math.log(per_ctx[n][0] * data[n][0].Lk) - 0.7 * b for n in ctxs if per_ctx[n][1]]
        a = math.exp(sum(la) / len(la)) if la else float("nan")
        emit({"keys": keys, "workload": "mla_decode", "stage": "fit", "b": float(f"{b:.6g}"),
              "a_sweep": float(f"{a_fit:.6g}"), "a_70": float(f"{a:.6g}"),
              "contexts_reaching_0.7_at_thr_le_1": [n for n in ctxs if per_ctx[n][1]]}, rows)
        for n in ctxs:
            w, call, skip_at, mask, out = data[n]
            kbytes = w.B * w.Lk * 576 * 2
            dense_ms = timer.ms(lambda: call(0.0))
            dense_out = out.clone()
            t70, reach, i70, ireach = per_ctx[n]
            cases = [("bisected", "chained", t70, reach)]
            if math.isfinite(a):
                cases.append(("calibrated", "chained") + calibrated_threshold(a, b, 0.7, w.Lk))
            cases.append(("bisected", "independent", i70, ireach))
            emit({"keys": keys, "workload": f"mla_decode_{n}k", "stage": "dense",
                  "ms": round(dense_ms, 4), "k_gbs": round(kbytes / dense_ms / 1e6, 1),
                  "frac_hbm": round(kbytes / dense_ms / 1e6 / HBM_PEAK_GBS, 4)}, rows)
            for kind, mode, thr, reach in cases:
                ms = timer.ms(lambda: call(thr, mode))
                s = skip_at(thr, mode)
                call(thr, mode)
                torch.cuda.synchronize()
                m = mask.cpu().numpy()
                keys_per_tile = np.full(m.shape[-1], 128)
                keys_per_tile[-1] = w.Lk - 128 * (m.shape[-1] - 1)
                kept_keys = int(((m == 0) * keys_per_tile[None, None, :]).sum())
                flops = 2.0 * w.Hq * (w.B * w.Lk * 576 + kept_keys * 512)
                emit({"keys": keys, "workload": f"mla_decode_{n}k", "stage": kind,
                      "split_mode": mode, "threshold": float(f"{thr:.6g}"), "reachable": reach,
                      "skip": round(s, 4), "ms": round(ms, 4),
                      "k_gbs": round(kbytes / ms / 1e6, 1),
                      "frac_hbm": round(kbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                      "mfma_tflops": round(flops / ms / 1e9, 1),
                      "frac_bf16_peak": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                      "speedup": round(dense_ms / ms, 3),
                      "rel_l2_vs_dense": float(f"{rel_l2_gpu(out, dense_out):.3e}")}, rows)
        del data
        torch.cuda.empty_cache()
    cols = ["keys", "workload", "stage", "split_mode", "threshold", "b", "a_70", "reachable",
            "skip", "ms", "k_gbs", "frac_hbm", "mfma_tflops", "frac_bf16_peak", "speedup",
            "rel_l2_vs_dense"]
    return rows, cols


# --------------------------------------------------------------------------- GQA decode

def run_decode(args):
    from synth import WORKLOADS, make_inputs

    timer, rows = Timer(), []
    w = WORKLOADS["gqa_decode_32k"]
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in "qkv")
    del x
    ws = torch.empty(ss_attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lk, w.D, w.Dv, 0),
                     dtype=torch.uint8, device="cuda")
    mask = torch.empty(mask_shape_decode(w.B, w.Hkv, w.Lk), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda")

    def part(thr):
        ss_attn_decode_partial(q, k, v, scale=w.scale, threshold=thr, skip_mask=mask,
                               workspace=ws)

    def call(thr):
        part(thr)
        ss_attn_decode_combine(q, k, ws, out, v=v)

    def skip_at(thr):
        part(thr)
        torch.cuda.synchronize()
        return skip_fraction(mask)

    kb = w.B * w.Hkv * w.Lk * w.D * 2
    dense_ms = timer.ms(lambda: call(0.0))
    dense_out = out.clone()
    emit({"workload": w.name, "target": 0.0, "threshold": 0.0, "skip": 0.0,
          "ms": round(dense_ms, 4), "gbs": round(2 * kb / dense_ms / 1e6, 1), "speedup": 1.0},
         rows)
    for tgt in (0.5, 0.7, 0.9):
        thr, s, reach = bisect_threshold(skip_at, tgt)
        ms = timer.ms(lambda: call(thr))
        s = skip_at(thr)
        by = kb * (1 + (1 - s))
        emit({"workload": w.name, "target": tgt, "threshold": float(f"{thr:.6g}"),
              "reachable": reach, "skip": round(s, 4), "ms": round(ms, 4),
              "gbs": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / HBM_PEAK_GBS, 4),
              "speedup": round(dense_ms / ms, 3),
              "rel_l2_vs_dense": float(f"{rel_l2_gpu(out, dense_out):.3e}")}, rows)
    cols = ["target", "threshold", "reachable", "skip", "ms", "gbs", "frac_hbm", "speedup",
            "rel_l2_vs_dense"]
    return rows, cols


# --------------------------------------------------------------------------- paged decode

def _paged_batch(timer, rows, name, seed, lens, Hq, Hkv, D, Dv, bs, r, latent):
    """Dense and ~70 % skip (one factor, threshold factor / L_b per sequence,
    bisected over the batch) for one paged batch; skip per length bucket."""
    from synth import paged_decode

    from . import ss_attn_decode_paged

    t = time.time()
    x = paged_decode(seed, lens, Hq, Hkv, D, Dv, 64 if not latent else 256, r, bs, latent=latent)
    log(f"[paged] {name}: generated {sum(lens)} tokens in {time.time() - t:.1f}s")
    q, kc = x["q"].cuda(), x["k_cache"].cuda()
    vc = None if latent else x["v_cache"].cuda()
    table, sl = x["block_table"].cuda(), x["seq_lens"].cuda()
    del x
    B, L = len(lens), max(lens)
    ws = torch.empty(ss_attn_decode_workspace_bytes(B, Hq, Hkv, L, D, Dv, 0), dtype=torch.uint8,
                     device="cuda")
    mask = torch.empty(mask_shape_decode(B, Hkv, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, Dv), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def call(factor):
        ss_attn_decode_paged(q, kc, vc, table, sl, max_seq_len=L, out=out,
                             dv=Dv if latent else None, scale=scale, factor=factor,
                             skip_mask=mask, workspace=ws)

    def skip_at(factor):
        call(factor)
        torch.cuda.synchronize()
        return skip_fraction(mask)

    nK = [-(-n // 128) for n in lens]
    kb = sum(lens) * Hkv * D * 2
    dense_bytes = kb if latent else kb + sum(lens) * Hkv * Dv * 2
    dense_ms = timer.ms(lambda: call(0.0))
    dense_out = out.clone()
    emit({"workload": name, "stage": "dense", "tokens": sum(lens), "ms": round(dense_ms, 4),
          "gbs": round(dense_bytes / dense_ms / 1e6, 1)}, rows)
    # skip is non-decreasing in the factor: bisect it in log space over the batch
    lo, hi = 1e-3, 1e6
    if skip_at(hi) < 0.7:
        factor = hi
    else:
        for _ in range(40):
            mid = math.sqrt(lo * hi)
            if skip_at(mid) < 0.7:
                lo = mid
            else:
                hi = mid
        factor = hi
    ms = timer.ms(lambda: call(factor))
    s = skip_at(factor)
    m = mask.cpu().numpy()
    kept_keys = 0
    per_bucket = {}
    width = 8192 if not latent else 16384
    for b, n in enumerate(lens):
        keys = np.full(nK[b], 128)
        keys[-1] = n - 128 * (nK[b] - 1)
        mb = m[b, :, :nK[b]]
        kept_keys += int(((mb == 0) * keys[None, :]).sum())
        lo_k = (n - 1) // width * (width // 1024)
        bucket = f"{lo_k}K-{lo_k + width // 1024}K"
        sk, vis = per_bucket.get(bucket, (0, 0))
        per_bucket[bucket] = (sk + int((mb == 1).sum()), vis + mb.size)
    # latent: V is inside K, skipping saves no bytes
    by = kb if latent else kb + kept_keys * Dv * 2
    emit({"workload": name, "stage": "sparse", "factor": float(f"{factor:.6g}"),
          "skip": round(s, 4), "ms": round(ms, 4), "gbs": round(by / ms / 1e6, 1),
          "frac_hbm": round(by / ms / 1e6 / HBM_PEAK_GBS, 4), "speedup": round(dense_ms / ms, 3),
          "rel_l2_vs_dense": float(f"{rel_l2_gpu(out, dense_out):.3e}")}, rows)
    for bucket in sorted(per_bucket, key=lambda k: int(k.split("K")[0])):
        sk, vis = per_bucket[bucket]
        emit({"workload": name, "stage": "skip by length", "bucket": bucket,
              "skip": round(sk / vis, 4)}, rows)
    del q, kc, vc, table, sl, ws, mask, out
    torch.cuda.empty_cache()


def run_paged(args):
    timer, rows = Timer(), []
    rng = np.random.default_rng(7000)
    lens = [int(x) for x in rng.integers(1024, 32769, size=32)]
    _paged_batch(timer, rows, "paged_decode_32seq", 7000, lens, 32, 8, 128, 128, 16, 3.0, False)
    # latent cache: 16 sequences of 4K-64K keys, 128 heads on one 576-wide
    # latent head, 64-key blocks
    rng = np.random.default_rng(7100)
    lens = [int(x) for x in rng.integers(4096, 65537, size=16)]
    _paged_batch(timer, rows, "paged_latent_decode_16seq", 7100, lens, 128, 1, 576, 512, 64, 3.0,
                 True)
    cols = ["workload", "stage", "tokens", "factor", "bucket", "skip", "ms", "gbs", "frac_hbm",
            "speedup", "rel_l2_vs_dense"]
    return rows, cols


# --------------------------------------------------------------------------- stability

def gumbel_closed_form_skip(L: int, a: float, tk: int = 128) -> float:
    """Expected skip fraction of one streaming pass over L keys with i.i.d.
    standard-Gumbel scaled scores at threshold a / L: the running max before
    tile j+1 is ln(tk j) plus a Gumbel draw, the tile max ln(tk) plus another,
    their difference is logistic, so tile j+1 is skipped with probability
    a j / (a j + L); the first tile never is."""
    n = L // tk
    j = np.arange(1, n)
    return float((a * j / (a * j + L)).sum() / n)


def run_stability(args):
    from synth import WORKLOADS, gumbel_decode, make_inputs

    timer, rows = Timer(), []
    base = WORKLOADS["gqa_decode_32k"]
    ctxs = [4096, 8192, 16384, 32768, 65536, 131072, 204800]
    for dist in ("clustered r=3", "clustered r=9", "gumbel"):
        data = {}
        for L in ctxs:
            B = max(1, min(64, (1 << 30) // (L * base.Hkv * base.D * 2)))
            seed = base.seed + 10 + ctxs.index(L)
            t = time.time()
            if dist == "gumbel":
                w = base.replace(B=B, Lk=L, seed=seed)
                x = gumbel_decode(seed, B, w.Hq, w.Hkv, L, w.D, w.Dv, w.scale)
            else:
                w = base.replace(B=B, Lk=L, r=float(dist[-1]), seed=seed)
                x = make_inputs(w)
            q, k, v = (x[n].cuda() for n in "qkv")
            del x
            ws = torch.empty(ss_attn_decode_workspace_bytes(B, w.Hq, w.Hkv, L, w.D, w.Dv, 0),
                             dtype=torch.uint8, device="cuda")
            mask = torch.empty(mask_shape_decode(B, w.Hkv, L), dtype=torch.uint8, device="cuda")
            out = torch.empty((B, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda")
            log(f"[stability] {dist} L={L} B={B} generated in {time.time() - t:.1f}s")

            def call(thr, q=q, k=k, v=v, ws=ws, mask=mask, out=out, w=w):
                ss_attn_decode_partial(q, k, v, scale=w.scale, threshold=thr, skip_mask=mask,
                                       workspace=ws)
                ss_attn_decode_combine(q, k, ws, out, v=v)

            def skip_at(thr, call=call, mask=mask):
                call(thr)
                torch.cuda.synchronize()
                return skip_fraction(mask)

            data[L] = (B, call, skip_at)
        for tgt in (0.7, 0.9):
            t32, s32, reach = bisect_threshold(data[32768][2], tgt, iters=30, tol=0.003)
            factor = t32 * 32768
            emit({"keys": dist, "target": tgt, "stage": "calibrated at 32K",
                  "threshold": float(f"{t32:.6g}"), "factor": float(f"{factor:.6g}"),
                  "skip": round(s32, 4), "reachable": reach}, rows)
            for L in ctxs:
                B, call, skip_at = data[L]
                thr_a = ss_resolve_threshold("direct", threshold=min(factor / L, 1.0), seqlen=L)
                clamped = factor / L > 1.0
                s_fixed = skip_at(t32)
                s_scaled = skip_at(thr_a)
                dense_ms = timer.ms(lambda: call(0.0), iters=7)
                ms = timer.ms(lambda: call(thr_a), iters=7)
                closed = (round(gumbel_closed_form_skip(L, thr_a * L), 4) if dist == "gumbel"
                          else None)
                emit({"keys": dist, "target": tgt, "L": L, "B": B,
                      "skip_fixed_threshold": round(s_fixed, 4),
                      "skip_factor_over_L": round(s_scaled, 4),
                      "closed_form_factor_over_L": closed,
                      "threshold_factor_over_L": float(f"{thr_a:.6g}"),
                      "factor_over_L_clamped_to_1": clamped,
                      "dense_ms": round(dense_ms, 4), "ms": round(ms, 4),
                      "speedup": round(dense_ms / ms, 3)}, rows)
        del data
        torch.cuda.empty_cache()
    cols = ["keys", "target", "stage", "L", "B", "threshold", "factor", "skip", "reachable",
            "skip_fixed_threshold", "skip_factor_over_L", "closed_form_factor_over_L",
            "threshold_factor_over_L", "factor_over_L_clamped_to_1", "dense_ms", "ms", "speedup"]
    return rows, cols


RUNS = {"prefill": run_prefill_sweep, "video": run_video, "latent": run_latent,
        "decode": run_decode, "paged": run_paged, "stability": run_stability}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("run", choices=sorted(RUNS))
    ap.add_argument("--out", default=None, help="also write a markdown table here")
    args = ap.parse_args(argv)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    lib()
    t = time.time()
    rows, cols = RUNS[args.run](args)
    log(f"[{args.run}] done in {time.time() - t:.1f}s")
    if args.out:
        cmd = "python -m block_sparse_attention_online_amd.harness " + " ".join(
            argv if argv is not None else sys.argv[1:])
        with open(args.out, "w") as f:
            f.write(f"# {args.run}\n\nCommand: `{cmd}`\n\n{md_table(rows, cols)}\n")


if __name__ == "__main__":
    main()
