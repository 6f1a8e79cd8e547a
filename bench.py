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
# VALU issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 fp32 VALU instruction per
# 4 cycles per SIMD (16 lanes, non-packed) -> 614.4 G wave-instructions/s.
VALU_PEAK_GIPS = 256 * 4 * 2.4 / 4


def pre_one_read(T: int, H: int) -> bool:
    """Whether the library's pre-map takes its one-read form at these sizes (the bench's
    buffers are 16-byte aligned and the machine's GPU is a 256-CU gfx950)."""
    return H % 8 == 0 and T >= 1024 and 1024 < H <= 8192


def pre_small_batch(T: int, H: int) -> bool:
    """Whether the library's pre-map takes its one-launch small-batch form (16-byte rows,
    1 <= T <= 192, H <= 8192, on a 256-CU gfx950)."""
    return H % 8 == 0 and 1 <= T <= 192 and H <= 8192


def sinkhorn_valu_per_wave(iters: int) -> int:
    """VALU instructions one wave of sinkhorn_kernel issues for its 64 matrices, counted
    in the compiled gfx950 code (iters >= 1): 141 outside the iteration loop (loads,
    softmax, the final scaling) plus 40 per iteration (4 row and 4 column scales, each
    one multiply, three FMAs and a reciprocal)."""
    return 141 + 40 * iters

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
    ap.add_argument("--only", default="all",
                    choices=["all", "pre", "post", "sinkhorn", "pre_dots", "post_bwd", "sinkhorn_bwd", "pre_dots_bwd",
                             "pre_bf16", "expand", "head", "head_mean", "pre_bwd", "post_project", "fused",
                             "post_pre", "f32", "pre_f32", "post_f32", "expand_f32", "head_mean_f32"],
                    help="run only one call in the timed loop (for profiling)")
    ap.add_argument("--presplit", action="store_true",
                    help="split the fixed weights once before timing and time mhc_pre_fused_presplit (a decode "
                         "loop's form: the weights do not change between steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-steady-state", action="store_true",
                    help="skip the steady-state sublayer step of the default run (for per-kernel profiles of the "
                         "headline step alone: both steps launch the collapse kernel)")
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="read a buffer of this many MiB before every timed rep (0: never); by default 512 "
                         "when a step moves less than 512 MB, so no rep starts with its data in the caches")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one captured HIP graph (no host launch cost)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU work (single-core seconds) of the oracle sample")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) turn two rocprofv3 --pmc CSV runs into the stored per-kernel HBM traffic")
    ap.add_argument("--traffic-command", default="", help="the profiling command, recorded with --write-traffic")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.write_traffic:
        _, T, H = WORKLOADS[args.workload]
        write_traffic(args.write_traffic[0], args.write_traffic[1], T, H, args.traffic_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the mHC path shards tokens with no exchange; "
              "no multi-GPU run is implemented here). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mhc_hyper_connection_amd as mhc
    from mhc_inputs import (algorithmic_bytes_expand_f32, algorithmic_bytes_head_mean_f32,
                            algorithmic_bytes_post_f32, algorithmic_bytes_pre_f32)
    from mhc_inputs import (algorithmic_bytes_expand, algorithmic_bytes_head, algorithmic_bytes_head_mean,
                            algorithmic_bytes_pre_bf16,
                            algorithmic_bytes_post, algorithmic_bytes_post_backward, algorithmic_bytes_pre,
                            algorithmic_bytes_pre_backward, algorithmic_bytes_pre_dots,
                            algorithmic_bytes_pre_dots_backward,
                            algorithmic_bytes_sinkhorn, algorithmic_bytes_sinkhorn_backward, external_dots,
                            layer_inputs, post_grad, pre_grads, sinkhorn_grad, sinkhorn_logits)

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
    if args.only in ("sinkhorn", "sinkhorn_bwd"):
        sk_logits = torch.from_numpy(sinkhorn_logits()).to(dev)
        sk_out = torch.empty_like(sk_logits)
    if args.only == "sinkhorn_bwd":
        sk_grad = torch.from_numpy(sinkhorn_grad()).to(dev)
    if args.only == "post_bwd":
        d_out = bf16(post_grad(T, H, cfg=cfg))
        d_x = torch.empty_like(x)
        d_res = torch.empty_like(res)
        d_post = torch.empty_like(post)
        d_comb = torch.empty_like(comb)

    if args.presplit:
        mhc.mhc_pre_split_weights(hc_fn, ws)  # once, outside the timed steps

    def call_pre():
        if args.presplit:
            mhc.mhc_pre_fused_presplit(res, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"],
                                       p["post_mult"], p["num_iters"], y=y, post=post, comb=comb, workspace=ws)
            return
        mhc.mhc_pre_fused(res, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"],
                          p["post_mult"], p["num_iters"], y=y, post=post, comb=comb, workspace=ws)

    def call_post():
        mhc.mhc_post(x, res, post, comb, out=out)

    dots = None
    if args.only == "pre_dots":
        # external projection logits of a realistic spread (|dot| ~ 0.02 * sqrt(4H)), one split,
        # the sum of squares computed from the streams
        g = np.random.default_rng(11)
        dots = torch.from_numpy((g.standard_normal((T, 24)) * 0.02 * math.sqrt(4 * H)).astype(np.float32)).to(dev)

    def call_pre_dots():
        mhc.mhc_pre_from_dots(dots, res, hc_scale, hc_base, None, None, p["rms_eps"], p["pre_eps"],
                              p["sinkhorn_eps"], p["post_mult"], p["num_iters"], y=y, post=post, comb=comb)

    if args.only == "pre_dots_bwd":
        g_dy, g_post, g_comb = pre_grads(T, H, cfg=cfg)
        g_dy = bf16(g_dy)
        g_post = torch.from_numpy(g_post).to(dev)
        g_comb = torch.from_numpy(g_comb).to(dev)
        bdots = torch.from_numpy(external_dots(T, H, cfg=cfg)[0]).to(dev)
        d_res_b = torch.empty_like(res)
        ws_b = torch.empty(max(mhc.mhc_pre_backward_workspace_bytes(T), 1), dtype=torch.uint8, device=dev)

    def call_pre_dots_bwd():
        mhc.mhc_pre_from_dots_backward(g_dy, g_post, g_comb, bdots, res, hc_scale, hc_base, None, None,
                                       p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"], p["post_mult"],
                                       p["num_iters"], d_res=d_res_b, workspace=ws_b)

    if args.only == "pre_bwd":
        f_dy, f_post, f_comb = pre_grads(T, H, cfg=cfg)
        f_dy = bf16(f_dy)
        f_post = torch.from_numpy(f_post).to(dev)
        f_comb = torch.from_numpy(f_comb).to(dev)
        f_dres = torch.empty_like(res)
        f_ws = torch.empty(max(mhc.mhc_pre_fused_backward_workspace_bytes(T, H), 1), dtype=torch.uint8, device=dev)

    def call_pre_bwd():
        mhc.mhc_pre_fused_backward(f_dy, f_post, f_comb, res, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"],
                                   p["sinkhorn_eps"], p["post_mult"], p["num_iters"], d_res=f_dres, workspace=f_ws)

    if args.only == "pre_bf16":
        hc_fn16 = hc_fn.to(torch.bfloat16)
    if args.only == "head":
        head_fn = hc_fn[:4].contiguous()
        head_scale = hc_scale[:1].contiguous()
        head_base = hc_base[:4].contiguous()
    if args.only == "expand":
        streams_out = torch.empty_like(res)

    def call_pre_bf16():
        mhc.mhc_pre_fused_bf16(res, hc_fn16, hc_scale, hc_base, p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"],
                               p["post_mult"], p["num_iters"], y=y, post=post, comb=comb, workspace=ws)

    def call_expand():
        mhc.mhc_expand(x, streams=streams_out)

    def call_head():
        mhc.mhc_head(res, head_fn, head_scale, head_base, p["rms_eps"], p["pre_eps"], y=y, workspace=ws)

    def call_head_mean():
        mhc.mhc_head_mean(res, y=y)

    def call_sinkhorn():
        mhc.mhc_sinkhorn(sk_logits, out=sk_out, num_iters=p["num_iters"], eps=p["sinkhorn_eps"])

    def call_sinkhorn_bwd():
        mhc.mhc_sinkhorn_backward(sk_grad, sk_logits, num_iters=p["num_iters"], eps=p["sinkhorn_eps"],
                                  d_logits=sk_out)

    def call_post_bwd():
        mhc.mhc_post_backward(d_out, x, res, post, comb, d_x=d_x, d_res=d_res, d_post=d_post, d_comb=d_comb)

    if args.only in ("f32", "pre_f32", "post_f32", "expand_f32", "head_mean_f32"):
        # fp32 residual streams [T, 4, H] (full fp32 N(0,1) values), the same weights and x
        from mhc_inputs import f32_streams
        res32 = torch.from_numpy(f32_streams(T, H, cfg)).to(dev)
        out32 = torch.empty_like(res32)

    def call_pre_f32():
        mhc.mhc_pre_fused_f32(res32, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"], p["sinkhorn_eps"],
                              p["post_mult"], p["num_iters"], y=y, post=post, comb=comb, workspace=ws)

    def call_post_f32():
        mhc.mhc_post_f32(x, res32, post, comb, out=out32)

    def call_expand_f32():
        mhc.mhc_expand_f32(x, streams=out32)

    def call_head_mean_f32():
        mhc.mhc_head_mean_f32(res32, y=y)

    if args.only in ("post_bwd", "post_f32"):
        call_pre()  # the forward's mixes (untimed)

    steady_state = args.only == "all" and H % 8 == 0 and not args.no_steady_state
    if args.only in ("post_project", "fused") or steady_state:
        # the post-map with the next sublayer's projection fused in (the next weights are
        # hc_fn again); "fused" is the steady-state sublayer step: the pre-map from the
        # previous post-map's dots, then the post-map updating the streams in place.  The
        # default run times it too, after the headline step, as a separate figure.
        pp_dm = torch.empty(T, 24, dtype=torch.float32, device=dev)
        pp_sq = torch.empty(T, dtype=torch.float32, device=dev)
        pp_ws = torch.empty(mhc.mhc_post_project_workspace_bytes(T, H), dtype=torch.uint8, device=dev)
        streams = res.clone()
        call_pre()  # mixes for the first post-map (untimed)
        mhc.mhc_post_project(x, streams, post, comb, hc_fn, out=out, dot_mix=pp_dm, sqrsum=pp_sq, workspace=pp_ws)

    def call_post_project():
        mhc.mhc_post_project(x, res, post, comb, hc_fn, out=out, dot_mix=pp_dm, sqrsum=pp_sq, workspace=pp_ws)

    def call_fused():
        mhc.mhc_pre_from_dots(pp_dm, streams, hc_scale, hc_base, pp_sq, None, p["rms_eps"], p["pre_eps"],
                              p["sinkhorn_eps"], p["post_mult"], p["num_iters"], y=y, post=post, comb=comb)
        mhc.mhc_post_project(x, streams, post, comb, hc_fn, out=streams, dot_mix=pp_dm, sqrsum=pp_sq,
                             workspace=pp_ws)

    if args.only == "post_pre" or steady_state:
        # the steady-state sublayer step in one call: the post-map and the next pre-map
        # (the next weights are hc_fn again), the streams updated in place; the mixes
        # alternate between two buffers, each call reading the previous call's
        pp2_ws = torch.empty(mhc.mhc_pre_fused_workspace_bytes(T, H), dtype=torch.uint8, device=dev)
        pp2_streams = res.clone()
        pp2_y = torch.empty_like(y)
        call_pre()  # mixes for the first post-map (untimed)
        pp2_mix = [(post.clone(), comb.clone()), (torch.empty_like(post), torch.empty_like(comb))]
        pp2_turn = [0]

    def call_post_pre():
        (pa, ca), (pb, cb) = pp2_mix[pp2_turn[0]], pp2_mix[1 - pp2_turn[0]]
        mhc.mhc_post_pre_fused(x, pp2_streams, pa, ca, hc_fn, hc_scale, hc_base, p["rms_eps"], p["pre_eps"],
                               p["sinkhorn_eps"], p["post_mult"], p["num_iters"], out=pp2_streams, y=pp2_y,
                               post_next=pb, comb_next=cb, workspace=pp2_ws)
        pp2_turn[0] = 1 - pp2_turn[0]

    def step():
        if args.only in ("all", "pre"):
            call_pre()
        if args.only in ("all", "post"):
            call_post()
        if args.only == "sinkhorn":
            call_sinkhorn()
        if args.only == "pre_dots":
            call_pre_dots()
        if args.only == "sinkhorn_bwd":
            call_sinkhorn_bwd()
        if args.only == "post_bwd":
            call_post_bwd()
        if args.only == "pre_dots_bwd":
            call_pre_dots_bwd()
        if args.only == "pre_bf16":
            call_pre_bf16()
        if args.only == "expand":
            call_expand()
        if args.only == "head":
            call_head()
        if args.only == "head_mean":
            call_head_mean()
        if args.only == "pre_bwd":
            call_pre_bwd()
        if args.only == "post_project":
            call_post_project()
        if args.only == "fused":
            call_fused()
        if args.only == "post_pre":
            call_post_pre()
        if args.only in ("f32", "pre_f32"):
            call_pre_f32()
        if args.only in ("f32", "post_f32"):
            call_post_f32()
        if args.only == "expand_f32":
            call_expand_f32()
        if args.only == "head_mean_f32":
            call_head_mean_f32()

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

    flush_buf = None

    def timed_reps(fn, n):
        """As timed(), or with the flush buffer read before each rep (HIP events around
        each rep only; the flush is not counted).  A read evicts the caches and leaves
        clean lines: a fill would leave dirty ones, written back during the timed rep."""
        if flush_buf is None:
            return timed(fn, n)
        torch.cuda.synchronize()
        evs = []
        for _ in range(n):
            flush_buf.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    run_step = step
    if args.graph:
        # capture one step on a side stream (after a warm-up there), then replay it
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()

    pre_b = algorithmic_bytes_pre(T, H)
    post_b = algorithmic_bytes_post(T, H)
    step_bytes = step_algorithmic_bytes(args.only, T, H, sk_logits)
    flush_mb = args.flush_mb if args.flush_mb >= 0 else (512 if step_bytes < 512 * 10 ** 6 else 0)
    if flush_mb > 0:
        flush_buf = torch.ones(flush_mb << 18, dtype=torch.float32, device=dev)
        flush_buf.sum()  # write back the fill's own dirty lines before timing
        torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps{' (graph replays)' if args.graph else ''}"
          f"{f', {flush_mb} MiB read before each' if flush_mb else ''}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ms_step = timed_reps(run_step, args.steps)
    wall = time.perf_counter() - t0

    breakdown = {}
    if args.only in ("all", "pre"):
        breakdown["pre_ms"] = timed_reps(call_pre, max(args.steps, 1))
    if args.only in ("all", "post"):
        breakdown["post_ms"] = timed_reps(call_post, max(args.steps, 1))
    if args.only == "sinkhorn":
        breakdown["sinkhorn_ms"] = ms_step
    if args.only == "pre_dots":
        breakdown["pre_dots_ms"] = ms_step
    if args.only == "sinkhorn_bwd":
        breakdown["sinkhorn_bwd_ms"] = ms_step
    if args.only == "post_bwd":
        breakdown["post_bwd_ms"] = ms_step
    if args.only == "pre_dots_bwd":
        breakdown["pre_dots_bwd_ms"] = ms_step
    for mode in ("pre_bf16", "expand", "head", "head_mean", "pre_bwd", "post_project", "fused", "post_pre", "expand_f32",
                 "head_mean_f32"):
        if args.only == mode:
            breakdown[mode + "_ms"] = ms_step
    if args.only in ("f32", "pre_f32"):
        breakdown["pre_f32_ms"] = timed_reps(call_pre_f32, max(args.steps, 1))
    if args.only in ("f32", "post_f32"):
        breakdown["post_f32_ms"] = timed_reps(call_post_f32, max(args.steps, 1))

    eff_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    steady = None
    if steady_state:
        # The same layer computed as a steady-state sublayer step, where a post-map is
        # followed by the next pre-map: as two calls (the pre-map (A1, A3-A5) from the dots
        # and sum of squares the previous post-map produced, then the post-map (A6) that also
        # computes the next pre-map's projection (A1-A2)), and as one call of
        # mhc_post_pre_fused.  Every row of the method runs once per step; a model's first
        # sublayer still needs mhc_pre_fused.
        print("[bench] timing the steady-state sublayer step", file=sys.stderr, flush=True)
        for _ in range(max(args.warmup, 1)):
            call_fused()
        ms_f = timed_reps(call_fused, max(args.steps, 1))
        eff_f = step_bytes / (ms_f * 1e-3) / 1e9
        two_calls = {"calls": "mhc_pre_from_dots (one split, sqrsum supplied) + mhc_post_project (in place)",
                     "ms_per_step": round(ms_f, 5), "tokens_per_s": round(T / (ms_f * 1e-3), 1),
                     "effective_GBps": round(eff_f, 1), "hbm_frac": round(eff_f / HBM_PEAK_GBPS, 4)}
        # the same step as one call: the post-map and the next pre-map fused (the library's
        # steady-state form; one launch where the one-read form applies)
        for _ in range(max(args.warmup, 1)):
            call_post_pre()
        ms_o = timed_reps(call_post_pre, max(args.steps, 1))
        eff_o = step_bytes / (ms_o * 1e-3) / 1e9
        steady = {"calls": "mhc_post_pre_fused (in place, the mixes alternating between two buffers)",
                  "ms_per_step": round(ms_o, 5), "tokens_per_s": round(T / (ms_o * 1e-3), 1),
                  "effective_GBps": round(eff_o, 1), "hbm_frac": round(eff_o / HBM_PEAK_GBPS, 4),
                  "algorithmic_bytes": step_bytes, "two_calls": two_calls}

    # Per-call rooflines.  mhc_post and mhc_sinkhorn are one kernel launch each;
    # mhc_pre_fused is one in its one-read form (16-byte rows, T >= 1024, 1024 < H <= 8192
    # on a 256-CU gfx950) and four otherwise (weight split, projection, slice sums, collapse).
    calls = {}
    proj = "pre_proj_stream_kernel" if H % 8 == 0 else "pre_proj_kernel"
    col = "pre_collapse_vec8_kernel" if H % 8 == 0 else "pre_collapse_scalar_kernel"
    # the two-pass form: the weight split (unless done before the steps), the projection, the
    # slice sums (above 64 tokens; below, the collapse sums the slices) and the collapse
    sums = [] if T <= 64 else ["pre_mixsum_kernel"]
    one_read = pre_one_read(T, H)
    small = pre_small_batch(T, H)
    pre_kernels = "pre_coop_kernel" if one_read else "pre_decode_kernel" if small else "+".join(
        ([] if args.presplit else ["pre_prep_kernel"]) + [proj] + sums + [col])
    split_kernels = "pre_coop_kernel" if one_read else "pre_decode_kernel" if small else "+".join(
        ["pre_prep_kernel", proj] + sums + [col])
    if "pre_ms" in breakdown:
        calls["mhc_pre_fused"] = (pre_kernels, breakdown["pre_ms"], pre_b)
    if "post_ms" in breakdown:
        calls["mhc_post"] = ("post_vec8_kernel" if H % 8 == 0 else "post_scalar_kernel", breakdown["post_ms"], post_b)
    if "sinkhorn_ms" in breakdown:
        calls["mhc_sinkhorn"] = ("sinkhorn_kernel", breakdown["sinkhorn_ms"], step_bytes)
    if "pre_dots_ms" in breakdown:
        calls["mhc_pre_from_dots"] = ("pre_dots_kernel", breakdown["pre_dots_ms"], step_bytes)
    if "sinkhorn_bwd_ms" in breakdown:
        calls["mhc_sinkhorn_backward"] = ("sinkhorn_bwd_kernel", breakdown["sinkhorn_bwd_ms"], step_bytes)
    if "post_bwd_ms" in breakdown:
        calls["mhc_post_backward"] = ("post_bwd_kernel", breakdown["post_bwd_ms"], step_bytes)
    if "pre_bf16_ms" in breakdown:
        calls["mhc_pre_fused_bf16"] = (split_kernels, breakdown["pre_bf16_ms"], step_bytes)
    if "head_ms" in breakdown:
        calls["mhc_head"] = (split_kernels, breakdown["head_ms"], step_bytes)
    if "pre_bwd_ms" in breakdown:
        calls["mhc_pre_fused_backward"] = ("pre_prep_kernel+" + proj + "+pre_mixsum_kernel+pre_dots_bwd_kernel+"
                                           "pre_bwd_partial_kernel+pre_bwd_final_kernel+proj_bwd_wfrag_kernel+"
                                           "proj_bwd_kernel+dw_reduce_kernel", breakdown["pre_bwd_ms"], step_bytes)
    if "expand_ms" in breakdown:
        calls["mhc_expand"] = ("expand_kernel", breakdown["expand_ms"], step_bytes)
    if "head_mean_ms" in breakdown:
        calls["mhc_head_mean"] = ("head_mean_kernel", breakdown["head_mean_ms"], step_bytes)
    if "pre_dots_bwd_ms" in breakdown:
        calls["mhc_pre_from_dots_backward"] = ("pre_dots_bwd_kernel+pre_bwd_partial_kernel+pre_bwd_final_kernel",
                                               breakdown["pre_dots_bwd_ms"], step_bytes)
    if "post_project_ms" in breakdown:
        calls["mhc_post_project"] = ("pre_prep_kernel+post_proj_stream_kernel+pre_mixsum_kernel",
                                     breakdown["post_project_ms"], step_bytes)
    if "pre_f32_ms" in breakdown:
        proj32 = "+".join(["pre_proj_f32s_kernel"] + sums + ["pre_collapse_f32s_kernel"])
        calls["mhc_pre_fused_f32"] = (proj32, breakdown["pre_f32_ms"], algorithmic_bytes_pre_f32(T, H))
    if "post_f32_ms" in breakdown:
        calls["mhc_post_f32"] = ("post_f32s_kernel", breakdown["post_f32_ms"], algorithmic_bytes_post_f32(T, H))
    if "expand_f32_ms" in breakdown:
        calls["mhc_expand_f32"] = ("expand_f32s_kernel", breakdown["expand_f32_ms"], step_bytes)
    if "head_mean_f32_ms" in breakdown:
        calls["mhc_head_mean_f32"] = ("head_mean_f32s_kernel", breakdown["head_mean_f32_ms"], step_bytes)
    if "post_pre_ms" in breakdown:
        post_k = "post_vec8_kernel" if H % 8 == 0 else "post_scalar_kernel"
        calls["mhc_post_pre_fused"] = ("pre_coop_kernel" if one_read else "pre_decode_kernel" if small
                                       else post_k + "+" + split_kernels,
                                       breakdown["post_pre_ms"], step_bytes)
    if "fused_ms" in breakdown:
        calls["mhc_pre_from_dots+mhc_post_project"] = (
            "pre_collapse_vec8_kernel+pre_prep_kernel+post_proj_stream_kernel+pre_mixsum_kernel", breakdown["fused_ms"],
            step_bytes)
    traffic = load_traffic(T, H, args.only)
    per_call = {}
    for name, (kern, ms_k, bytes_k) in calls.items():
        achieved = bytes_k / (ms_k * 1e-3) / 1e9
        per_call[name] = {"kernel": kern, "avg_ms": round(ms_k, 5), "algorithmic_bytes": bytes_k,
                          "achieved": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBPS, 4),
                          "traffic": call_traffic(traffic, kern)}
    # The dominant kernel: the longest single kernel launch of the step.  At
    # T=8192, H=7168 that is the post-map (one launch, 64% of the bytes); at the
    # decode shape the small-batch pre-map.  Calls of several launches (the two-pass
    # pre-map) are not single kernels; the post-map stands in for them.
    single = {k: v for k, v in per_call.items() if "+" not in v["kernel"]}
    dom = max(single, key=lambda k: single[k]["avg_ms"]) if single else next(iter(per_call))
    if "mhc_post" in per_call and any("+" in v["kernel"] for v in per_call.values()):
        dom = "mhc_post"
    d = per_call[dom]
    roofline = {"bound": "hbm", "achieved": d["achieved"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": d["frac"], "traffic": d["traffic"], "kernel": d["kernel"], "call": dom,
                "avg_ms": d["avg_ms"], "algorithmic_bytes": d["algorithmic_bytes"]}
    if dom == "mhc_sinkhorn":
        # one lane per matrix: bound by VALU issue, not by its 128 B per matrix
        waves = sk_logits.shape[0] // 64
        instr = waves * sinkhorn_valu_per_wave(p["num_iters"])
        achieved = instr / (d["avg_ms"] * 1e-3) / 1e9
        roofline = {"bound": "alu", "achieved": round(achieved, 1), "peak": VALU_PEAK_GIPS,
                    "unit": "G wave64 VALU instructions/s", "frac": round(achieved / VALU_PEAK_GIPS, 4),
                    "traffic": d["traffic"], "kernel": d["kernel"], "call": dom, "avg_ms": d["avg_ms"],
                    "valu_instructions": instr, "hbm": {"achieved": d["achieved"], "peak": HBM_PEAK_GBPS,
                                                        "unit": "GB/s"}}

    # Sanity figures: the launch floor of the step's kernel count (one-element fills,
    # launched the same way), and what a plain elementwise copy sustains here.
    one_launch = pre_one_read(T, H) or pre_small_batch(T, H)
    npre = 1 if one_launch else 2 + (0 if args.presplit else 1) + (0 if T <= 64 else 1)
    npre32 = 2 + (0 if T <= 64 else 1)
    nker = {"all": npre + 1, "pre": npre, "post": 1, "post_project": 3, "fused": 4,
            "post_pre": 1 if one_launch else 1 + npre + (1 if args.presplit else 0),
            "f32": npre32 + 1,
            "pre_f32": npre32, "post_f32": 1}.get(args.only)
    launch_floor_ms = None
    if nker:
        one = torch.zeros(1, device=dev)

        def floor_step():
            for _ in range(nker):
                one.fill_(0.0)
        launch_floor_ms = timed(floor_step, max(args.steps, 1))
    nc = 1 << 29
    csrc = torch.empty(nc, dtype=torch.bfloat16, device=dev).normal_()
    cdst = torch.empty_like(csrc)
    torch.neg(csrc, out=cdst)  # the first call loads the kernel
    ms_c = timed(lambda: torch.neg(csrc, out=cdst), 10)
    copy_gbps = round(4 * nc / (ms_c * 1e-3) / 1e9, 1)
    del csrc, cdst

    copy_cal = None
    if args.copy_calibration:
        # A plain elementwise kernel of known size (reads 1 GiB, writes 1 GiB): the
        # reference that scales the HBM byte counters of the kernels above.
        n = 1 << 29
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # the first call loads the kernel
        ms_copy = timed(lambda: torch.neg(src, out=dst), 5)
        copy_cal = {"kernel": "torch.neg (bf16, 2^29 elements)", "bytes_read": 2 * n, "bytes_written": 2 * n,
                    "ms": round(ms_copy, 4), "GBps": round(4 * n / (ms_copy * 1e-3) / 1e9, 1)}

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
        "dtype": "f32" if args.only.endswith("f32") or args.only == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": (f"mhc {args.only} 2^20 4x4 matrices" if args.only.startswith("sinkhorn") else
                                f"mhc {args.only if args.only != 'all' else 'pre+post'} T={T} H={H} HC=4"),
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "weights": "split once before the timed steps" if args.presplit else "split in every step",
                   "cache_flush_mib": flush_mb,
                   "T": T, "H": H, "hc": 4, "num_iters": p["num_iters"], "inputs": "resident in HBM"},
        "effective_GBps": round(eff_gbps, 1),
        "hbm_frac": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "breakdown_ms": {k: round(v, 5) for k, v in breakdown.items()},
        "roofline": roofline,
        "calls": per_call,
        "cpu_baseline": cpu,
        "launch_floor_ms": None if launch_floor_ms is None else round(launch_floor_ms, 5),
        "kernels_per_step": nker,
        "copy_GBps": copy_gbps,
        "steady_state": steady,
        "wall_s_timed": round(wall, 3),
    }
    if copy_cal:
        line["copy_calibration"] = copy_cal
    print(json.dumps(line), flush=True)


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mhc_hyper_connection_amd", "csrc")


def sources_digest() -> str:
    """sha256 over the HIP sources (name + bytes), to tell whether stored counters are stale."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_path(T: int, H: int) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_T{T}_H{H}.json")


def step_algorithmic_bytes(only: str, T: int, H: int, sk_logits) -> int:
    """What one timed step must move (each tensor counted once)."""
    from mhc_inputs import (algorithmic_bytes_expand_f32, algorithmic_bytes_head_mean_f32,
                            algorithmic_bytes_post_f32, algorithmic_bytes_pre_f32)
    from mhc_inputs import (algorithmic_bytes_expand, algorithmic_bytes_head, algorithmic_bytes_head_mean,
                            algorithmic_bytes_post, algorithmic_bytes_post_backward, algorithmic_bytes_pre,
                            algorithmic_bytes_pre_backward, algorithmic_bytes_pre_bf16, algorithmic_bytes_pre_dots,
                            algorithmic_bytes_pre_dots_backward, algorithmic_bytes_sinkhorn,
                            algorithmic_bytes_sinkhorn_backward, algorithmic_bytes_post_project)
    per_mode = {
        "post_project": lambda: algorithmic_bytes_post_project(T, H),
        "post_pre": lambda: algorithmic_bytes_pre(T, H) + algorithmic_bytes_post(T, H),
        "fused": lambda: algorithmic_bytes_pre_dots(T, H, splits=1, sqrsum=True) + algorithmic_bytes_post_project(T, H),
        "sinkhorn": lambda: algorithmic_bytes_sinkhorn(sk_logits.shape[0]),
        "sinkhorn_bwd": lambda: algorithmic_bytes_sinkhorn_backward(sk_logits.shape[0]),
        "post_bwd": lambda: algorithmic_bytes_post_backward(T, H),
        "pre_dots_bwd": lambda: algorithmic_bytes_pre_dots_backward(T, H),
        "pre_bf16": lambda: algorithmic_bytes_pre_bf16(T, H),
        "expand": lambda: algorithmic_bytes_expand(T, H),
        "head": lambda: algorithmic_bytes_head(T, H),
        "head_mean": lambda: algorithmic_bytes_head_mean(T, H),
        "pre_bwd": lambda: algorithmic_bytes_pre_backward(T, H),
        "pre_dots": lambda: algorithmic_bytes_pre_dots(T, H),
        "pre": lambda: algorithmic_bytes_pre(T, H),
        "post": lambda: algorithmic_bytes_post(T, H),
        "all": lambda: algorithmic_bytes_pre(T, H) + algorithmic_bytes_post(T, H),
        "f32": lambda: algorithmic_bytes_pre_f32(T, H) + algorithmic_bytes_post_f32(T, H),
        "pre_f32": lambda: algorithmic_bytes_pre_f32(T, H),
        "post_f32": lambda: algorithmic_bytes_post_f32(T, H),
        "expand_f32": lambda: algorithmic_bytes_expand_f32(T, H),
        "head_mean_f32": lambda: algorithmic_bytes_head_mean_f32(T, H),
    }
    return per_mode[only]()


def load_traffic(T: int, H: int, mode: str):
    """Per-kernel HBM bytes per launch in bench mode `mode`, from the stored counter runs,
    or None when they are missing or were taken on different kernel sources.  Counters
    are kept per mode: one kernel can move different bytes in different calls (the
    per-token reverse writes d_res on its own, only per-token values inside the fused
    reverse)."""
    try:
        with open(traffic_path(T, H)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest():
        return None
    kernels = rec.get("modes", {}).get(mode)
    if not kernels:
        return None
    return {k: v["bytes"] for k, v in kernels.items()}


def call_traffic(traffic, kernels: str):
    """Summed HBM bytes of the '+'-joined kernels of one call, if all were measured."""
    if not traffic:
        return None
    names = kernels.split("+")
    if not all(n in traffic for n in names):
        return None
    return sum(traffic[n] for n in names)


def _pmc_per_kernel(csv_dir: str, counter: str):
    """Mean counter value (KiB) per dispatch, by kernel, from a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    import re
    vals = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                m = re.search(r"(\w+_kernel)\b", row["Kernel_Name"]) or re.search(r"([A-Za-z_]\w*)", row["Kernel_Name"])
                name = m.group(1)
                if "neg_kernel" in row["Kernel_Name"] or ("neg" in row["Kernel_Name"] and "elementwise" in row["Kernel_Name"]):
                    name = "calibration_copy"
                vals.setdefault(name, []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def write_traffic(fetch_dir: str, write_dir: str, T: int, H: int, command: str) -> None:
    """Turn two sets of rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; one
    subdirectory per bench mode) into bytes per launch, per mode and kernel, each counter
    scaled by what it reads for the calibration copy kernel of the same run."""
    cal_bytes = 2 * (1 << 29)
    modes, cals = {}, {}
    for mode in sorted(os.listdir(fetch_dir)):
        fd, wd = os.path.join(fetch_dir, mode), os.path.join(write_dir, mode)
        if not (os.path.isdir(fd) and os.path.isdir(wd)):
            continue
        fetch = _pmc_per_kernel(fd, "FETCH_SIZE")
        write = _pmc_per_kernel(wd, "WRITE_SIZE")
        if "calibration_copy" not in fetch or "calibration_copy" not in write:
            continue
        f_fetch = cal_bytes / (fetch["calibration_copy"] * 1024)
        f_write = cal_bytes / (write["calibration_copy"] * 1024)
        cals[mode] = {"fetch_kib": round(fetch["calibration_copy"], 1), "write_kib": round(write["calibration_copy"], 1),
                      "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}
        kernels = {}
        for k in sorted(set(fetch) & set(write)):
            if k == "calibration_copy":
                continue
            rb, wb = fetch[k] * 1024 * f_fetch, write[k] * 1024 * f_write
            kernels[k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                          "read_bytes": round(rb), "write_bytes": round(wb), "bytes": round(rb + wb)}
        modes[mode] = kernels
    rec = {"workload": f"T={T} H={H}", "command": command, "counters": ["FETCH_SIZE", "WRITE_SIZE"],
           "calibration": {"kernel": "torch.neg bf16 2^29 elements", "bytes_read": cal_bytes,
                           "bytes_written": cal_bytes, "per_mode": cals},
           "sources_sha256": sources_digest(), "modes": modes}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(T, H), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


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
    # when the whole batch is less CPU work than the target, repeat it
    reps = max(1, int(round(target_s / max(n * per_tok, 1e-9))))
    print(f"[bench] cpu baseline: {reps} x {n} tokens on {threads} threads", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(reps):
            list(ex.map(lambda k: run(k * chunk, (k + 1) * chunk), range(threads)))
    wall = time.perf_counter() - t0
    # one thread, about 3 CPU-seconds
    n1 = int(min(T, max(1, 3.0 / max(per_tok, 1e-9))))
    t1 = time.perf_counter()
    run(0, n1)
    wall1 = time.perf_counter() - t1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": round(reps * n / wall, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread": {"value": round(n1 / wall1, 2), "unit": "tokens/s", "sample": f"{n1} tokens"},
            "cpu_model": model, "logical_cpus": os.cpu_count(),
            "sample": (f"{reps} pass{'es' if reps > 1 else ''} over {n} of {T} tokens of the T={T} H={H} pre+post "
                       f"step, fp64 oracle, {threads} threads (about {reps * n * per_tok:.0f} CPU-seconds)"),
            "wall_s": round(wall, 2)}


if __name__ == "__main__":
    main()
