#!/usr/bin/env python3
"""Benchmark of the mHC pre-map + post-map on one MI355X.

One step = mhc_pre_fused (RMS, 24 x 4H projection, sigmoid mixes, Sinkhorn,
collapse) followed by mhc_post (x plays the sublayer output) on T=8192 tokens,
H=7168, HC=4, seeded synthetic inputs already resident in HBM.

Prints one JSON line: tokens/s for the whole step, effective HBM bandwidth
(algorithmic bytes / time), the roofline of the dominant kernel measured with
HIP events on the stream the kernels run on, and the CPU oracle's throughput on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "mHC pre+post tokens/s and effective HBM GB/s (% of peak), T=8192 H=7168"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published

WORKLOADS = {
    # name: (cfg id, T, H)
    "layer_h7168": (3, 8192, 7168),
    "post_h4096": (2, 4096, 4096),
    "ragged_h1000": (6, 3000, 1000),
    "decode_h7168": (5, 32, 7168),
    "tiny": (1, 16, 256),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer_h7168", choices=sorted(WORKLOADS))
    ap.add_argument("--only", default="all", choices=["all", "pre", "post", "sinkhorn"],
                    help="run only one call in the timed loop (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the mHC path shards tokens with no exchange; "
              "no multi-GPU run is implemented here). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mhc_hyper_connection_amd as mhc
    from mhc_inputs import (algorithmic_bytes_post, algorithmic_bytes_pre, algorithmic_bytes_sinkhorn, layer_inputs,
                            sinkhorn_logits)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mhc.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg, T, H = WORKLOADS[args.workload]
    print(f"[bench] generating inputs {args.workload} T={T} H={H}", file=sys.stderr, flush=True)
    inp = layer_inputs(T, H, cfg=cfg)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    res = bf16(inp.res)
    x = bf16(inp.x)
    hc_fn = torch.from_numpy(inp.hc_fn).to(dev)
    hc_scale = torch.from_numpy(inp.hc_scale).to(dev)
    hc_base = torch.from_numpy(inp.hc_base).to(dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    post = torch.empty(T, 4, dtype=torch.float32, device=dev)
    comb = torch.empty(T, 4, 4, dtype=torch.float32, device=dev)
    out = torch.empty(T, 4, H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(mhc.mhc_pre_fused_workspace_bytes(T, H), 1), dtype=torch.uint8, device=dev)
    p = inp.params
    sk_logits = None
    if args.only == "sinkhorn":
        sk_logits = torch.from_numpy(sinkhorn_logits()).to(dev)
        sk_out = torch.empty_like(sk_logits)

    def call_pre():
        mhc.mhc_pre_fused(res, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"],
                          p["post_mult"], p["num_iters"], y=y, post=post, comb=comb, workspace=ws)

    def call_post():
        mhc.mhc_post(x, res, post, comb, out=out)

    def call_sinkhorn():
        mhc.mhc_sinkhorn(sk_logits, out=sk_out, num_iters=p["num_iters"], eps=p["sinkhorn_eps"])

    def step():
        if args.only in ("all", "pre"):
            call_pre()
        if args.only in ("all", "post"):
            call_post()
        if args.only == "sinkhorn":
            call_sinkhorn()

    stream = torch.cuda.current_stream(dev)

    def timed(fn, n):
        """Average ms per call of fn over n calls, HIP events on the kernels' stream."""
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ms_step = timed(step, args.steps)
    wall = time.perf_counter() - t0

    pre_b = algorithmic_bytes_pre(T, H)
    post_b = algorithmic_bytes_post(T, H)
    breakdown = {}
    if args.only in ("all", "pre"):
        breakdown["pre_ms"] = timed(call_pre, max(args.steps, 1))
    if args.only in ("all", "post"):
        breakdown["post_ms"] = timed(call_post, max(args.steps, 1))
    if args.only == "sinkhorn":
        breakdown["sinkhorn_ms"] = ms_step

    if args.only == "sinkhorn":
        step_bytes = algorithmic_bytes_sinkhorn(sk_logits.shape[0])
    else:
        step_bytes = (pre_b if args.only in ("all", "pre") else 0) + (post_b if args.only in ("all", "post") else 0)
    eff_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    # Roofline of the dominant call (largest share of the step).
    cand = []
    if "pre_ms" in breakdown:
        cand.append(("mhc_pre_fused", breakdown["pre_ms"], pre_b))
    if "post_ms" in breakdown:
        cand.append(("mhc_post", breakdown["post_ms"], post_b))
    if "sinkhorn_ms" in breakdown:
        cand.append(("mhc_sinkhorn", breakdown["sinkhorn_ms"], step_bytes))
    name, ms_k, bytes_k = max(cand, key=lambda c: c[1])
    achieved = bytes_k / (ms_k * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": name,
                "avg_ms": round(ms_k, 5), "algorithmic_bytes": bytes_k}

    copy_cal = None
    if args.copy_calibration:
        n = 1 << 29  # 1 GiB of bf16
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        ms_copy = timed(lambda: dst.copy_(src), 5)
        copy_cal = {"bytes_read": 2 * n, "bytes_written": 2 * n, "ms": round(ms_copy, 4),
                    "GBps": round(4 * n / (ms_copy * 1e-3) / 1e9, 1)}

    cpu = None
    if not args.no_cpu_baseline and args.only in ("all",):
        cpu = cpu_baseline(inp, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"mhc {args.only if args.only != 'all' else 'pre+post'} T={T} H={H} HC=4",
                   "T": T, "H": H, "hc": 4, "num_iters": p["num_iters"], "inputs": "resident in HBM"},
        "effective_GBps": round(eff_gbps, 1),
        "hbm_frac": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "breakdown_ms": {k: round(v, 5) for k, v in breakdown.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    if copy_cal:
        line["copy_calibration"] = copy_cal
    print(json.dumps(line), flush=True)


def cpu_baseline(inp, target_s: float):
    """The fp64 oracle, as it stands, on a bounded token sample of the same workload (threads over tokens)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    threads = max(1, min(os.cpu_count() or 1, 16))
    T, H = inp.T, inp.H
    p = inp.params

    def run(lo, hi):
        r = oracle.pre(inp.res[lo:hi], inp.hc_fn, inp.hc_scale, inp.hc_base, p["rms_eps"], p["pre_eps"],
                       p["sinkhorn_eps"], p["post_mult"], p["num_iters"])
        oracle.post(inp.x[lo:hi], inp.res[lo:hi], r["post"], r["comb"])

    print("[bench] cpu baseline: calibrating", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    run(0, 4)
    per_tok = (time.perf_counter() - t0) / 4
    n = int(min(T, max(threads, target_s / max(per_tok, 1e-9))))
    n = max(threads, (n // threads) * threads)
    chunk = n // threads
    print(f"[bench] cpu baseline: {n} tokens on {threads} threads", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda k: run(k * chunk, (k + 1) * chunk), range(threads)))
    wall = time.perf_counter() - t0
    return {"value": round(n / wall, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {T} tokens of the T={T} H={H} pre+post step, fp64 oracle, {threads} threads",
            "wall_s": round(wall, 2)}


if __name__ == "__main__":
    main()
