#!/usr/bin/env python3
"""Benchmark of the skip-softmax attention hot path on one MI355X.

Metric: prefill TFLOP/s + decode KV GB/s at ~70 % tile skip, and the speedup
over the same kernels at threshold 0 (dense).

One step is one split-KV decode call (decode kernel + log-sum-exp combine,
chained splits, so the skip decisions are those of one streaming pass) on
the GQA decode workload with the Llama-3.1-8B attention shape: batch 16, 32
query heads over 8 KV heads, head dim 128, 32768 cached keys, bf16 K/V
resident in HBM.  The threshold is calibrated first (bisection on the
kernel's own skip mask) to the target skip fraction.  ``value`` is the
decode's algorithmic bytes (K, plus V of the kept tiles, plus q and out) per
second of step wall time.  The causal GQA prefill (B1, Hq32/Hkv8, L16384,
D128) is timed in the same run and reported under ``prefill``.

Every timed step is preceded by a read of a 1 GiB buffer, so no step finds
K/V in L2 or in the 256 MB last-level cache (a read, not a rewrite: a rewrite
leaves dirty lines whose write-back to HBM would land inside the timed step);
the step and its kernels are
timed with HIP events on the stream they run on, and ``value`` uses the mean
of those step times.  ``warm_value`` is the same decode run back to back
(wall clock over the steps, caches left as the previous step left them).

``roofline`` is for the decode kernel alone: its algorithmic bytes (K, the V
of kept tiles, q) over its mean event time; the split partials it writes are
reported beside them, not counted.  ``rel_l2_vs_dense`` of every leg is the
output's relative L2 distance from the same kernels at threshold 0.  Every
chained decode checks that no look-back wait gave up.  ``decode_wide_gap`` is
the same decode on keys with a wide score gap (r = 9), where ~70 % skip comes
at a small threshold and a small error.  ``cpu_baseline`` times the fp64 CPU
oracle on a bounded sample of the same decode.  ``video`` is the non-causal
video-DiT attention (B1 H24, 32760 tokens) at the calibrated threshold of
target 0.7 and under timestep gating; ``latent`` the latent-cache decode
(B8, 128 heads, 576-wide rows, 131072 keys); ``backward`` the skip-aware
backward of the causal GQA prefill.

Usage: python bench.py [--steps K] [--warmup W] [--target-skip 0.7]
       python bench.py --copy-probe       (a plain 1 GiB device copy, for
                                           scaling hardware byte counters)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s + decode KV GB/s at ~70% tile skip; speedup vs dense"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gqa_traffic.json")
# the decode kernel's device code: its source and the device helpers it includes
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_online_amd", "csrc", f)
               for f in ("decode_gqa.hip", "device_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------- decode

def decode_bytes(mask_np, B, Hq, Hkv, Lk, D, Dv, S):
    """Algorithmic bytes of one decode call: K always; V of kept tiles; q; out;
    and (for the decode kernel alone) the split partials it writes."""
    import numpy as np

    nK = mask_np.shape[-1]
    keys = np.full(nK, 128, dtype=np.int64)
    keys[-1] = Lk - 128 * (nK - 1)
    kept_keys = int(((mask_np == 0) * keys[None, None, :]).sum())
    k_bytes = B * Hkv * Lk * D * 2
    v_bytes = kept_keys * Dv * 2
    q_bytes = B * Hq * D * 2
    out_bytes = B * Hq * Dv * 2
    part_bytes = S * B * Hq * (Dv + 1) * 4
    return {"k": k_bytes, "v_kept": v_bytes, "q": q_bytes, "out": out_bytes,
            "partials": part_bytes, "v_dense": B * Hkv * Lk * Dv * 2}


def rel_l2(torch, a, b) -> float:
    a, b = a.float(), b.float()
    return float(torch.linalg.norm(a - b) / torch.linalg.norm(b))


def bench_decode(ss, torch, args, r=None):
    from block_sparse_attention_online_amd.calibrate import bisect_threshold, skip_fraction
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS["gqa_decode_32k"]
    if r is not None:
        w = w.replace(r=r)
    t = time.time()
    x = make_inputs(w)
    log(f"[decode] generated {w.name} in {time.time() - t:.1f}s")
    q, k, v = (x[n].cuda() for n in "qkv")
    B, Hq, Hkv, Lk, D, Dv = w.B, w.Hq, w.Hkv, w.Lk, w.D, w.Dv
    S = ss.ss_decode_num_splits(B, Hq, Hkv, Lk, D, Dv)
    # zeroed once: its last 256 bytes count look-back waits that gave up
    ws = torch.zeros(ss.ss_attn_decode_workspace_bytes(B, Hq, Hkv, Lk, D, Dv, 0),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, Dv), dtype=torch.bfloat16, device="cuda")
    mask = torch.empty(ss.mask_shape_decode(B, Hkv, Lk), dtype=torch.uint8, device="cuda")

    def partial(thr):
        ss.ss_attn_decode_partial(q, k, v, scale=w.scale, threshold=thr, skip_mask=mask,
                                  workspace=ws)

    def combine():
        ss.ss_attn_decode_combine(q, k, ws, out, v=v)

    def skip_at(thr):
        partial(thr)
        torch.cuda.synchronize()
        return skip_fraction(mask)

    fixed = args.threshold if r is None else args.wide_threshold
    if fixed is not None:
        thr, reachable = fixed, True
    else:
        thr, _, reachable = bisect_threshold(skip_at, args.target_skip)
    log(f"[decode r={w.r:g}] threshold {thr:.6g} (reachable={reachable}) splits={S}")

    def timed(th, steps, warmup):
        """(step ms, decode kernel ms, combine ms) over `steps` cold steps, each
        after a cache-evicting read; plus the warm wall-clock step ms."""
        for _ in range(warmup):
            partial(th)
            combine()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i, e in enumerate(evs):
            evict_caches(args.flush)
            e[0].record()
            partial(th)
            e[1].record()
            combine()
            e[2].record()
        torch.cuda.synchronize()
        step = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
        kern = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        comb = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        t0 = time.perf_counter()
        for _ in range(steps):
            partial(th)
            combine()
        torch.cuda.synchronize()
        warm = (time.perf_counter() - t0) * 1e3 / steps
        return step, kern, comb, warm

    res = {"workload": w, "S": S, "thr": thr, "reachable": reachable, "x": x}
    if not args.only_sparse_decode:
        res["dense"] = timed(0.0, args.steps, args.warmup)
        dense_out = out.clone()
        log(f"[decode r={w.r:g}] dense: step {res['dense'][0]:.4f} ms, kernel "
            f"{res['dense'][1]:.4f} ms, warm step {res['dense'][3]:.4f} ms")
    res["sparse"] = timed(thr, args.steps, args.warmup)
    torch.cuda.synchronize()
    # every chained split of every call since the workspace was zeroed (the
    # bisection's, the dense and the sparse timed ones) found its
    # predecessors' maxima
    res["lookback_timeouts"] = ss.ss_attn_decode_lookback_timeouts(q, k, ws, v=v)
    assert res["lookback_timeouts"] == 0, \
        f"{res['lookback_timeouts']} look-back waits gave up: decisions not those of one pass"
    if not args.only_sparse_decode:
        res["rel_l2_vs_dense"] = rel_l2(torch, out, dense_out)
    res["mask"] = mask.cpu().numpy()
    res["skip"] = skip_fraction(mask)
    res["bytes"] = decode_bytes(res["mask"], B, Hq, Hkv, Lk, D, Dv, S)
    log(f"[decode r={w.r:g}] sparse: step {res['sparse'][0]:.4f} ms, kernel "
        f"{res['sparse'][1]:.4f} ms, combine {res['sparse'][2]:.4f} ms, warm step "
        f"{res['sparse'][3]:.4f} ms, skip {res['skip']:.3f}")
    return res


# --------------------------------------------------------------------------- prefill

def prefill_flops(mask_np, D, Dv):
    """Executed MFMA flops: 2*128*128*D per visited (query tile, key tile) for
    Q.K^T, plus 2*128*128*Dv per kept tile for P.V (full tiles as issued)."""
    visited = int((mask_np != 2).sum())
    kept = int((mask_np == 0).sum())
    return 2 * 128 * 128 * D * visited + 2 * 128 * 128 * Dv * kept, visited, kept


def bench_prefill(ss, torch, args, r, order):
    from block_sparse_attention_online_amd.calibrate import bisect_threshold, skip_fraction
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS["gqa_prefill_16k"].replace(r=r)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in "qkv")
    out = torch.empty_like(q)
    mask = torch.empty(ss.mask_shape_prefill(w.B, w.Hq, w.Lq, w.Lk), dtype=torch.uint8,
                       device="cuda")

    def run(thr):
        ss.ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=True, threshold=thr,
                              skip_mask=mask, order=order)

    def skip_at(thr):
        run(thr)
        torch.cuda.synchronize()
        return skip_fraction(mask)

    if args.prefill_threshold is not None:
        thr, reachable = args.prefill_threshold, True
    else:
        thr, s, reachable = bisect_threshold(skip_at, args.target_skip, iters=20, tol=0.01)

    def timed(th):
        for _ in range(max(2, args.warmup // 2)):
            run(th)
        torch.cuda.synchronize()
        steps = max(5, args.steps // 2)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i, e in enumerate(evs):
            evict_caches(args.flush)
            e[0].record()
            run(th)
            e[1].record()
        torch.cuda.synchronize()
        ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        return ms, mask.cpu().numpy()

    dense_ms, dmask = timed(0.0)
    dense_out = out.clone()
    sparse_ms, smask = timed(thr)
    err = rel_l2(torch, out, dense_out)
    fl_d, vis, _ = prefill_flops(dmask, w.D, w.Dv)
    fl_s, _, kept = prefill_flops(smask, w.D, w.Dv)
    fa = 4.0 * w.B * w.Hq * w.Lq * w.Lk * w.D * 0.5
    res = {"generator": f"clustered tile r={r:g}, {w.n_c} centroids", "order": order,
           "threshold": thr, "threshold_reaches_target": reachable,
           "skip_fraction": round(float((smask == 1).sum() / vis), 4),
           "ms": round(sparse_ms, 4), "dense_ms": round(dense_ms, 4),
           "speedup_vs_dense": round(dense_ms / sparse_ms, 3),
           "tflops_executed": round(fl_s / sparse_ms / 1e9, 2),
           "dense_tflops_executed": round(fl_d / dense_ms / 1e9, 2),
           "frac_of_bf16_peak": round(fl_s / sparse_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
           "dense_frac_of_bf16_peak": round(fl_d / dense_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
           "fa_convention_tflops": round(fa / sparse_ms / 1e9, 2),
           "rel_l2_vs_dense": float(f"{err:.3e}")}
    log(f"[prefill r={r} {order}] {res}")
    return res


# --------------------------------------------------------------------------- video DiT

def bench_video(ss, torch, args):
    """Non-causal video-DiT self-attention (B1 H24, 13x42x60 = 32760 latent
    tokens, D128, smooth-field generator).  Per visit order, the calibrated
    factor a*exp(b*s) is fitted on replicate 1 (a sweep of thresholds, least
    squares of ln(threshold*L) = ln a + b*s over the points with 2-98 % skip);
    replicate 0 is then timed dense, at the calibrated threshold of target
    0.7 (clamped to 1), and under timestep gating (dense until t <= 0.7) at
    t = 1.0 (dense) and t = 0.6 (sparse)."""
    import numpy as np

    from block_sparse_attention_online_amd.calibrate import (calibrated_threshold, fit_factor,
                                                             skip_fraction)
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS["video_dit_32760"]
    L = w.Lk
    grid = [float(f"{t:.3g}") for t in np.logspace(-6, 0, 13)]
    mask = torch.empty(ss.mask_shape_prefill(w.B, w.Hq, w.Lq, w.Lk), dtype=torch.uint8,
                       device="cuda")

    def load(seed):
        x = make_inputs(w.replace(seed=seed))
        return tuple(x[n].cuda() for n in "qkv")

    q, k, v = load(w.seed + 1)
    out = torch.empty_like(q)
    fits = {}
    for order in ("ascending", "diag_first"):
        pts = []
        for thr in grid:
            ss.ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=False, threshold=thr,
                                  skip_mask=mask, order=order)
            torch.cuda.synchronize()
            s = skip_fraction(mask)
            if 0.02 < s < 0.98:
                pts.append((thr, L, s))
        fits[order] = fit_factor(pts)
    del q, k, v
    q, k, v = load(w.seed)
    fa = 4.0 * w.B * w.Hq * w.Lq * w.Lk * w.D
    res = {"workload": "video_dit_32760 (B1 H24, 13x42x60 tokens, D128, non-causal)",
           "calibration": "a*exp(b*s) fitted on replicate 1, timed on replicate 0"}
    for order in ("ascending", "diag_first"):
        a, b = fits[order]

        def timed(th):
            for _ in range(2):
                ss.ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=False, threshold=th,
                                      skip_mask=mask, order=order)
            steps = max(3, args.steps // 10)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for e in evs:
                evict_caches(args.flush)
                e[0].record()
                ss.ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=False, threshold=th,
                                      skip_mask=mask, order=order)
                e[1].record()
            torch.cuda.synchronize()
            return sum(e[0].elapsed_time(e[1]) for e in evs) / steps, mask.cpu().numpy()

        dense_ms, dmask = timed(0.0)
        dense_out = out.clone()
        thr, reachable = calibrated_threshold(a, b, 0.7, L)
        ms, smask = timed(thr)
        err = rel_l2(torch, out, dense_out)
        fl_d, vis, _ = prefill_flops(dmask, w.D, w.Dv)
        fl_s, _, kept = prefill_flops(smask, w.D, w.Dv)
        gating = []
        for t in (1.0, 0.6):
            thr_t, _ = calibrated_threshold(a, b, 0.7, L, timestep=t, disabled_until=0.7)
            ms_t, m_t = timed(thr_t)
            gating.append({"timestep": t, "disabled_until": 0.7,
                           "mode": "dense" if thr_t == 0 else "sparse",
                           "threshold": float(f"{thr_t:.6g}"), "ms": round(ms_t, 3),
                           "skip_fraction": round(float((m_t == 1).sum() / vis), 4)})
        res[order] = {"a": float(f"{a:.6g}"), "b": float(f"{b:.6g}"), "target": 0.7,
                      "threshold": float(f"{thr:.6g}"), "threshold_reaches_target": reachable,
                      "skip_fraction": round(float((smask == 1).sum() / vis), 4),
                      "ms": round(ms, 3), "dense_ms": round(dense_ms, 3),
                      "speedup_vs_dense": round(dense_ms / ms, 3),
                      "tflops_executed": round(fl_s / ms / 1e9, 1),
                      "frac_of_bf16_peak": round(fl_s / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                      "dense_tflops_executed": round(fl_d / dense_ms / 1e9, 1),
                      "dense_frac_of_bf16_peak": round(fl_d / dense_ms / 1e9 / BF16_PEAK_TFLOPS,
                                                       4),
                      "fa_convention_tflops": round(fa / ms / 1e9, 1),
                      "rel_l2_vs_dense": float(f"{err:.3e}"), "gating": gating}
        log(f"[video {order}] {res[order]}")
    return res


# --------------------------------------------------------------------------- prefill backward

def bench_backward(ss, torch, args):
    """Skip-aware backward of the causal GQA prefill (B1 Hq32 Hkv8 L16384
    D128, clustered tile generator r=3): the forward at the threshold runs
    once, untimed, for the skip mask and lse; then the backward is timed
    replaying that mask, against the same backward with no mask (every
    visible tile: dense attention's gradients).  Algorithmic flops: the five
    products of a kept 128x128 tile pair (S, dP, dV, dK, dQ), 2*128*128*D
    each; the kernels run seven (S and dP are recomputed for dQ)."""
    from synth import WORKLOADS, make_inputs, output_gradient

    w = WORKLOADS["gqa_prefill_16k"]
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in "qkv")
    do = output_gradient(9, w.B, w.Hq, w.Lq, w.Dv).cuda()
    out = torch.empty_like(q)
    mask = torch.empty(ss.mask_shape_prefill(w.B, w.Hq, w.Lq, w.Lk), dtype=torch.uint8,
                       device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ss.ss_attn_prefill_backward_workspace_bytes(w.B, w.Hq, w.Lq),
                     dtype=torch.uint8, device="cuda")
    thr = args.backward_threshold
    ss.ss_attn_prefill_ex(q, k, v, out, scale=w.scale, causal=True, threshold=thr,
                          skip_mask=mask, lse=lse, order="diag_first")
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    visited, kept = int((m != 2).sum()), int((m == 0).sum())

    def timed(use_mask):
        def run():
            ss.ss_attn_prefill_backward(q, k, v, out, do, lse, mask if use_mask else None,
                                        scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv,
                                        workspace=ws)
        for _ in range(max(2, args.warmup // 4)):
            run()
        torch.cuda.synchronize()
        steps = max(5, args.steps // 5)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            evict_caches(args.flush)
            e[0].record()
            run()
            e[1].record()
        torch.cuda.synchronize()
        return sum(e[0].elapsed_time(e[1]) for e in evs) / steps

    dense_ms = timed(False)
    ms = timed(True)
    per_pair = 5 * 2 * 128 * 128 * w.D
    tf = per_pair * kept / ms / 1e9
    tf_d = per_pair * visited / dense_ms / 1e9
    res = {"workload": "gqa_prefill_16k (B1 Hq32 Hkv8 L16384 D128 causal), clustered tile "
                       "r=3, dO ~ N(0,1)",
           "threshold": thr, "order": "diag_first",
           "skip_fraction": round(1 - kept / visited, 4),
           "ms": round(ms, 4), "dense_ms": round(dense_ms, 4),
           "speedup_vs_dense": round(dense_ms / ms, 3),
           "tflops_algorithmic": round(tf, 1), "dense_tflops_algorithmic": round(tf_d, 1),
           "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
           "tflops_executed": round(tf * 7 / 5, 1)}
    log(f"[backward] {res}")
    return res


# --------------------------------------------------------------------------- latent decode

def bench_latent(ss, torch, args):
    """Latent-cache decode at 131072 keys: threshold 0 against the threshold
    bisected to the target skip, with chained splits (score pass, then the
    kept tiles) and with independent splits (one streaming pass per split);
    K bytes per second."""
    from block_sparse_attention_online_amd.calibrate import bisect_threshold, skip_fraction
    from synth import WORKLOADS, make_inputs
    import numpy as np

    w = WORKLOADS["mla_decode_128k"]
    x = make_inputs(w)
    q, k = x["q"].cuda(), x["k"].cuda()
    del x
    ws = torch.zeros(ss.ss_attn_decode_workspace_bytes(w.B, w.Hq, 1, w.Lk, 576, 512, 0),
                     dtype=torch.uint8, device="cuda")
    mask = torch.empty(ss.mask_shape_decode(w.B, 1, w.Lk), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, 512), dtype=torch.bfloat16, device="cuda")

    def call(thr, mode):
        ss.ss_attn_decode_partial(q, k, None, dv=512, scale=w.scale, threshold=thr,
                                  skip_mask=mask, workspace=ws, split_mode=mode)
        ss.ss_attn_decode_combine(q, k, ws, out, dv=512)

    def skip_at(thr, mode):
        call(thr, mode)
        torch.cuda.synchronize()
        return skip_fraction(mask)

    def timed(th, mode):
        for _ in range(3):
            call(th, mode)
        steps = max(5, args.steps // 4)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i, e in enumerate(evs):
            evict_caches(args.flush)
            e[0].record()
            call(th, mode)
            e[1].record()
        torch.cuda.synchronize()
        return sum(e[0].elapsed_time(e[1]) for e in evs) / steps

    kbytes = w.B * w.Lk * 576 * 2
    dense_flops = 2.0 * w.Hq * w.B * w.Lk * (576 + 512)
    dense_ms = timed(0.0, "chained")
    dense_out = out.clone()

    def leg(mode, fixed):
        if fixed is not None:
            thr, reachable = fixed, True
        else:
            thr, _, reachable = bisect_threshold(lambda t: skip_at(t, mode), args.target_skip,
                                                 iters=24, tol=0.005)
        ms = timed(thr, mode)
        err = rel_l2(torch, out, dense_out)
        s = skip_at(thr, mode)
        m = mask.cpu().numpy()
        nK = m.shape[-1]
        keys = np.full(nK, 128, dtype=np.int64)
        keys[-1] = w.Lk - 128 * (nK - 1)
        kept_keys = int(((m == 0) * keys[None, None, :]).sum())
        # MFMA work: Q.K^T over every key (576 wide), P.V over kept keys (512 wide)
        flops = 2.0 * w.Hq * (w.B * w.Lk * 576 + kept_keys * 512)
        return {"split_mode": mode, "threshold": thr, "threshold_reaches_target": reachable,
                "skip_fraction": round(s, 4), "ms": round(ms, 4),
                "k_gbs": round(kbytes / ms / 1e6, 1),
                "frac_of_hbm_peak": round(kbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                "mfma_tflops": round(flops / ms / 1e9, 1),
                "frac_of_bf16_peak": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                "speedup_vs_dense": round(dense_ms / ms, 3),
                "rel_l2_vs_dense": float(f"{err:.3e}")}

    res = {"workload": f"{w.name} (B8 Hq128, one 576-wide latent head, value = first 512 "
                       "columns)",
           "dense_ms": round(dense_ms, 4), "dense_k_gbs": round(kbytes / dense_ms / 1e6, 1),
           "dense_frac_of_hbm_peak": round(kbytes / dense_ms / 1e6 / HBM_PEAK_GBS, 4),
           "dense_frac_of_bf16_peak": round(dense_flops / dense_ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
    res.update(leg("chained", args.latent_threshold))
    res["independent"] = leg("independent", None)
    log(f"[latent] {res}")
    return res


# --------------------------------------------------------------------------- CPU baseline

def cpu_baseline(dec, seconds):
    """The fp64 oracle on the same decode (all sequences, same threshold),
    repeated until about ``seconds`` of CPU time."""
    import oracle

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} "
                             f"({os.path.basename(i.get('filepath', ''))})" for i in info)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    w, x = dec["workload"], dec["x"]
    reps, t0 = 0, time.perf_counter()
    while True:
        # chained splits decide as one streaming pass: the oracle's single split
        res = oracle.decode(x["q"], x["k"], x["v"], w.scale, dec["thr"], 1)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or reps >= 50:
            break
    by = decode_bytes(res["mask"], w.B, w.Hq, w.Hkv, w.Lk, w.D, w.Dv, dec["S"])
    tot = by["k"] + by["v_kept"] + by["q"] + by["out"]
    return {"value": round(tot * reps / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "host_cpu_count": os.cpu_count(), "cpu_model": model,
            "blas": blas,
            "threads_note": "cores = BLAS threads; the oracle's per-tile loop is Python, so "
                            "only its matrix products use more than one thread",
            "sample": f"the whole decode call ({w.B * w.Hkv} (batch, kv head) pairs, same "
                      f"threshold, one streaming pass as the chained splits decide) run "
                      f"{reps}x in {dt:.1f} s of fp64 numpy"}


# --------------------------------------------------------------------------- main

def evict_caches(buf):
    """Push K/V out of L2 and the last-level cache before a timed call by
    READING a 1 GiB buffer.  Rewriting it (fill_) would leave up to the cache's
    size of dirty lines behind, and their write-back to HBM would then be
    charged to the next timed call."""
    buf.max()


def copy_probe(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))


def traffic_entry(launch_bytes):
    """HBM bytes per decode launch from committed hardware-counter runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--target-skip", type=float, default=0.70)
    ap.add_argument("--threshold", type=float, default=None,
                    help="use this decode threshold instead of calibrating")
    ap.add_argument("--prefill-threshold", type=float, default=None,
                    help="use this prefill threshold instead of calibrating")
    ap.add_argument("--wide-threshold", type=float, default=None,
                    help="use this threshold for the wide-gap (r=9) decode leg")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-wide-decode", action="store_true")
    ap.add_argument("--no-video", action="store_true")
    ap.add_argument("--no-latent", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only-sparse-decode", action="store_true",
                    help="time only the sparse decode (for hardware-counter runs)")
    ap.add_argument("--only-latent", action="store_true",
                    help="time only the latent decode (for kernel-trace runs)")
    ap.add_argument("--latent-threshold", type=float, default=None,
                    help="use this latent-decode threshold instead of calibrating")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the skip-aware prefill backward")
    ap.add_argument("--backward-threshold", type=float, default=1.0,
                    help="forward threshold whose skip mask the backward replays")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_online_amd as ss

    ss.lib()
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.only_sparse_decode:
        args.no_prefill = args.no_cpu = args.no_latent = args.no_backward = True
        args.no_wide_decode = args.no_video = True
    args.flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    if args.only_latent:
        print(json.dumps({"latent": bench_latent(ss, torch, args)}), flush=True)
        return
    if args.only_backward:
        print(json.dumps({"backward": bench_backward(ss, torch, args)}), flush=True)
        return

    dec = bench_decode(ss, torch, args)
    w, by = dec["workload"], dec["bytes"]
    wall, kern, comb, warm = dec["sparse"]
    step_bytes = by["k"] + by["v_kept"] + by["q"] + by["out"]
    # the decode kernel's algorithmic bytes: K, the V of kept tiles and q (the
    # call's out is written by the merge); the split partials it writes are
    # implementation traffic, reported beside it, not counted
    kern_bytes = by["k"] + by["v_kept"] + by["q"]
    achieved = kern_bytes / (kern * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_entry(kern_bytes),
            "kernel": "decode_gqa_kernel<128,4>", "kernel_ms": round(kern, 4),
            "algorithmic_bytes_per_launch": kern_bytes,
            "split_partial_bytes_per_launch": by["partials"]}
    line = {
        "metric": METRIC,
        "value": round(step_bytes / (wall * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "warm_value": round(step_bytes / (warm * 1e-3) / 1e9, 1),
        "warm_ms_per_step": round(warm, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "kv_len": w.Lk, "head_dim": w.D, "generator":
                   f"clustered keys r={w.r:g}, {w.n_c} centroids, query near 1-3 centroids",
                   "threshold": dec["thr"], "threshold_reaches_target": dec["reachable"],
                   "skip_fraction": round(dec["skip"], 4), "num_splits": dec["S"],
                   "split_mode": "chained"},
        "roofline": roof,
        "lookback_timeouts": dec["lookback_timeouts"],
    }
    if "dense" in dec:
        dwall, dkern, _, dwarm = dec["dense"]
        line["speedup_vs_dense"] = round(dwall / wall, 3)
        line["dense_ms_per_step"] = round(dwall, 4)
        dense_bytes = by["k"] + by["v_dense"] + by["q"] + by["out"]
        line["dense_value"] = round(dense_bytes / (dwall * 1e-3) / 1e9, 1)
        line["rel_l2_vs_dense"] = float(f"{dec['rel_l2_vs_dense']:.3e}")
    if not args.no_wide_decode:
        wd = bench_decode(ss, torch, args, r=9.0)
        wb = wd["bytes"]
        wwall, wkern = wd["sparse"][0], wd["sparse"][1]
        wstep = wb["k"] + wb["v_kept"] + wb["q"] + wb["out"]
        wkb = wb["k"] + wb["v_kept"] + wb["q"]
        line["decode_wide_gap"] = {
            "generator": f"clustered keys r=9, {wd['workload'].n_c} centroids",
            "threshold": wd["thr"], "threshold_reaches_target": wd["reachable"],
            "skip_fraction": round(wd["skip"], 4), "ms_per_step": round(wwall, 4),
            "gbs": round(wstep / (wwall * 1e-3) / 1e9, 1),
            "kernel_gbs": round(wkb / (wkern * 1e-3) / 1e9, 1),
            "kernel_frac_of_hbm_peak": round(wkb / (wkern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "dense_ms_per_step": round(wd["dense"][0], 4),
            "speedup_vs_dense": round(wd["dense"][0] / wwall, 3),
            "rel_l2_vs_dense": float(f"{wd['rel_l2_vs_dense']:.3e}"),
            "lookback_timeouts": wd["lookback_timeouts"]}
        del wd
    if not args.no_prefill:
        line["prefill"] = {"workload": "gqa_prefill_16k (B1 Hq32 Hkv8 L16384 D128 causal)",
                           "literal": bench_prefill(ss, torch, args, 3.0, "diag_first"),
                           "wide_gap": bench_prefill(ss, torch, args, 9.0, "diag_first")}
    if not args.no_video:
        line["video"] = bench_video(ss, torch, args)
    if not args.no_latent:
        line["latent"] = bench_latent(ss, torch, args)
    if not args.no_backward:
        line["backward"] = bench_backward(ss, torch, args)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(dec, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
