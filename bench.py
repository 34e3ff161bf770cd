#!/usr/bin/env python3
"""Throughput of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config IDX] [--pass fwd|bwd]

A step is one fa_fwd call (every kernel of the forward pass, including the
key-split merge when the library splits) over one batch of synthetic inputs
that are resident in HBM before timing starts. W untimed warm-up steps run
first, then more untimed steps for --warmup-seconds (clock ramp-up), then
exactly K timed steps (HIP events on the launch stream bracket them; their
mean is roofline.kernel_ms), then 100 more steps (20 backward) each
bracketed by its own events, whose median and minimum are
roofline.per_step_events. The default workload is the
bf16 causal GQA configuration (B=2, H=32, HKV=8, S=4096, D=128), the one the
headline metric is quoted on. Prints one JSON line.

Metric: TFLOP/s counting 4*B*H*D*sum_i |visible keys of row i| (masked
pairs are not counted), i.e. the two matrix products of attention restricted
to the mask. With --pass bwd a step is one backward pass (fa_bwd, on O and
LSE from one forward pass made before timing) and the count is 10*D per
visible pair (the five products of the backward pass).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (published)
# Published fp32 vector peak: 256 flop per clock per CU x 256 CUs x 2.4 GHz = 157.3 TFLOP/s.
# It counts packed fp32 FMAs; code built without them (as this library is) tops out at half.
PEAK_VALU_F32 = 157.3
KERNEL_SOURCES = [os.path.join(ROOT, "attention_forward_online_fa_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_fwd_common.h", "fa_api.cpp", "fa_kernels.h",
                            "fa_tile.h")]


def row_counts(wl: W.Workload, i: np.ndarray, mask_bh=None) -> np.ndarray:
    """|visible(i)| for query rows i of one (b, h): the causal / window key
    range [lo, hi), intersected with the visible blocks of a block mask."""
    i = np.asarray(i, dtype=np.int64)
    hi = np.minimum(i + 1, wl.Sk) if wl.causal else np.full(len(i), wl.Sk, np.int64)
    lo = np.maximum(i - wl.window + 1, 0) if wl.window > 0 else np.zeros(len(i), np.int64)
    if mask_bh is None:
        return np.maximum(hi - lo, 0)
    c0 = np.arange(mask_bh.shape[1], dtype=np.int64) * W.MASK_BLOCK_K       # block key ranges
    c1 = np.minimum(c0 + W.MASK_BLOCK_K, wl.Sk)
    inter = np.maximum(np.minimum(c1[None, :], hi[:, None]) - np.maximum(c0[None, :], lo[:, None]), 0)
    return (inter * (mask_bh[i // W.MASK_BLOCK_Q] != 0)).sum(axis=1)


def counted_flops(wl: W.Workload, block_mask=None) -> float:
    """4 D flop per visible (query, key) pair over every (b, h)."""
    i = np.arange(wl.Sq, dtype=np.int64)
    if block_mask is None:
        return 4.0 * wl.B * wl.H * wl.D * float(row_counts(wl, i).sum())
    total = 0.0
    g = wl.H // wl.HKV
    for b in range(wl.B):
        for h in range(wl.H):
            mb = 0 if block_mask.shape[0] == 1 else b
            mh = h if block_mask.shape[1] == wl.H else (h // g if block_mask.shape[1] > 1 else 0)
            total += float(row_counts(wl, i, block_mask[mb, mh]).sum())
    return 4.0 * wl.D * total


def algorithmic_bytes(wl: W.Workload) -> int:
    esz = 4 if wl.dtype == "f32" else 2
    q = wl.B * wl.H * wl.Sq * wl.D * esz
    kv = 2 * wl.B * wl.HKV * wl.Sk * wl.D * esz
    return q + kv + q + wl.B * wl.H * wl.Sq * 4


def per_step_events(step, stream, n: int) -> dict:
    """Median and minimum of n steps each bracketed by its own pair of HIP
    events on the launch stream (after the timed region; not part of it)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return {"n": n, "median_ms": round(float(np.median(ms)), 5), "min_ms": round(ms[0], 5)}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(wl: W.Workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    none exist or the kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def device_inputs(inp, torch):
    return W.device_tensors(inp, torch, "cuda")


def bench_backward(args, wl, inp, q, k, v, torch, fa):
    """Time the backward pass (fa_bwd; fa_bwd_strided on token-major workloads,
    fa_bwd_block_sparse under a block mask); prints one JSON line."""
    stream = torch.cuda.current_stream()
    scale = wl.scale()
    bmask = W.device_mask(inp, torch, "cuda")
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=scale,
                    block_mask=bmask)
    g, bits = W.make_grad_output(inp)
    if bits is not None:
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        src = torch.from_numpy(bits.view(np.int16)).view(tdt)
    else:
        src = torch.from_numpy(g)
    do = torch.empty_like(o)        # o's layout: token-major workloads stay token-major
    do.copy_(src.cuda())

    def step():
        fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window, scale=scale,
               stream=stream, block_mask=bmask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter() + args.warmup_seconds
    while time.perf_counter() < t_warm:
        step()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    per_step = per_step_events(step, stream, 20)
    flops = 2.5 * counted_flops(wl, inp.block_mask)          # 10 D per visible pair
    # MFMA backward kernels, except where the library's plan picks the per-row
    # VALU kernels (fp32 at D = 16, 48, 80 on small problems)
    plan = fa.bwd_plan(wl.B, wl.H, wl.HKV, wl.Sq, wl.Sk, wl.D,
                       torch.cuda.get_device_properties(0).multi_processor_count,
                       causal=bool(wl.causal), window=wl.window, dtype=wl.dtype)
    if not plan["per_row"]:
        bound, peak = "mfma", PEAK_TFLOPS[wl.dtype]
    else:
        bound, peak = "alu", PEAK_VALU_F32
    rec = {
        "metric": "attention bwd TFLOP/s (unmasked FLOPs, 10*D per visible pair), 1xMI355X",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "pass": "bwd", "B": wl.B, "H": wl.H, "HKV": wl.HKV,
                   "Sq": wl.Sq, "Sk": wl.Sk, "D": wl.D, "causal": wl.causal,
                   "window": wl.window, "layout": wl.layout,
                   "block_mask": None if inp.block_mask is None else list(inp.block_mask.shape),
                   "counted_flops": flops, "parallelism": "single GPU"},
        "roofline": {"bound": bound, "achieved": round(flops / (ev_ms * 1e-3) / 1e12, 3),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / (ev_ms * 1e-3) / 1e12 / peak, 4),
                     "per_step_events": per_step,
                     "traffic": None, "kernel_ms": round(ev_ms, 5)},
    }
    if args.cpu_rows > 0:
        # the oracle's backward on one (batch, kv-head group) slice of the workload
        from oracle import attention_backward
        gsz = wl.H // wl.HKV
        sl = W.small(wl, B=1, H=gsz, HKV=1)
        m = inp.block_mask
        if m is not None:   # the slice's mask: batch 0, the group's heads
            m = m[:1, :gsz] if m.shape[1] == wl.H else m[:1, :1]
        t1 = time.perf_counter()
        attention_backward(inp.q[:1, :gsz], inp.k[:1, :1], inp.v[:1, :1], g[:1, :gsz],
                           scale, bool(wl.causal), wl.window, block_mask=m)
        dt = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": round(2.5 * counted_flops(sl, m) / dt / 1e12, 6),
                               "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle",
                               "sample": f"batch 0, kv head 0 and its {gsz} query heads, fp64 "
                                         f"numpy, {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


def cpu_baseline(wl: W.Workload, inp, target_rows: int):
    """The fp64 oracle on a bounded row sample of the same workload."""
    from oracle import attention_rows
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(wl.seed + 7)
    total = wl.B * wl.H * wl.Sq
    flat = np.sort(rng.choice(total, size=min(target_rows, total), replace=False))
    rows = np.stack([flat // (wl.H * wl.Sq), (flat // wl.Sq) % wl.H, flat % wl.Sq], axis=1)
    bm = inp.block_mask
    if bm is None:
        flops = 4.0 * wl.D * float(row_counts(wl, rows[:, 2]).sum())
    else:
        g = wl.H // wl.HKV
        flops = 0.0
        bh = rows[:, 0] * wl.H + rows[:, 1]
        for key in np.unique(bh):
            b, h = int(key // wl.H), int(key % wl.H)
            mb = 0 if bm.shape[0] == 1 else b
            mh = h if bm.shape[1] == wl.H else (h // g if bm.shape[1] > 1 else 0)
            flops += 4.0 * wl.D * float(row_counts(wl, rows[bh == key, 2], bm[mb, mh]).sum())
    t0 = time.perf_counter()
    attention_rows(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window, rows,
                   block_mask=bm)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{len(rows)} random query rows of {total} (all heads), fp64 numpy, "
                      f"{dt:.2f} s; value counts the same unmasked FLOPs per row"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="after the W warm-up steps, keep running untimed steps until this "
                         "much time has passed (the GPU clock ramps up for about a second)")
    ap.add_argument("--config", type=int, default=W.HEADLINE)
    ap.add_argument("--num-splits", type=int, default=0, help="0 = the library's choice")
    ap.add_argument("--cpu-rows", type=int, default=262144,
                    help="rows of the CPU-oracle sample (0 = skip the CPU leg)")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="fwd: the forward pass (default); bwd: the backward pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device-to-device copy of MIB "
                         "MiB (reference for scaling HBM byte counters)")
    ap.add_argument("--gemm-ceiling", type=int, default=0, metavar="N",
                    help="instead of attention, time a dense bf16 N x N x N product "
                         "(torch.matmul, i.e. hipBLASLt) for reference: what the chip "
                         "sustains on dense bf16 matrix work under its power limit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_forward_online_fa_amd as fa

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": max(args.steps, 1)}), flush=True)
        return

    if args.gemm_ceiling:
        n = args.gemm_ceiling
        g = torch.Generator(device="cpu").manual_seed(1)
        a = torch.randn(n, n, generator=g).to(torch.bfloat16).cuda()
        b = torch.randn(n, n, generator=g).to(torch.bfloat16).cuda().t().contiguous()
        c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(max(args.warmup, 1)):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        t_warm = time.perf_counter() + args.warmup_seconds
        while time.perf_counter() < t_warm:
            torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"metric": "dense bf16 GEMM TFLOP/s (torch.matmul), reference only",
                          "n": n, "ms_per_gemm": round(ms, 5), "tflops": round(tf, 1),
                          "frac_of_bf16_peak": round(tf / PEAK_TFLOPS["bf16"], 4),
                          "steps": args.steps}), flush=True)
        return

    wl = W.CONFIGS[args.config]
    inp = W.make_inputs(wl)
    q, k, v = device_inputs(inp, torch)
    bmask = W.device_mask(inp, torch, "cuda")
    if args.which == "bwd":
        bench_backward(args, wl, inp, q, k, v, torch, fa)
        return
    o = torch.empty_like(q)          # q's layout (token-major workloads: token-major o)
    lse = torch.empty((wl.B, wl.H, wl.Sq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    scale = wl.scale()
    splits = fa.plan_splits(wl.B, wl.H, wl.HKV, wl.Sq, wl.Sk, wl.D, causal=bool(wl.causal),
                            window=wl.window, dtype=wl.dtype) if args.num_splits == 0 else args.num_splits

    def step():
        fa.fwd_into(q, k, v, o, lse, causal=bool(wl.causal), window=wl.window, scale=scale,
                    num_splits=args.num_splits, stream=stream, block_mask=bmask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter() + args.warmup_seconds
    while time.perf_counter() < t_warm:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps          # HIP events on the launch stream
    ms_per_step = wall * 1e3 / args.steps
    per_step = per_step_events(step, stream, 100)

    flops = counted_flops(wl, inp.block_mask)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    traffic = measured_traffic(wl)

    rec = {
        "metric": "attention fwd TFLOP/s (unmasked FLOPs) + % of MFMA peak, 1xMI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "HKV": wl.HKV, "Sq": wl.Sq,
                   "Sk": wl.Sk, "D": wl.D, "causal": wl.causal, "window": wl.window,
                   "layout": wl.layout, "block_mask": wl.mask or None,
                   "num_splits": splits, "counted_flops": flops,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel_ms": round(ev_ms, 5),
                     "per_step_events": per_step,
                     "algorithmic_bytes": algorithmic_bytes(wl)},
    }
    if args.cpu_rows > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_rows)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
