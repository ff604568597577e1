"""Benchmark of the multi-LoRA apply hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload ("bgmv_decode_x128"): the BGMV decode batch of 64 tokens,
rank 16, 4096 -> 4096, 32 resident slots, ids ~ finite Zipf(1.1), applied to
128 module instances (for example q, k, v, o of 32 layers) in one launch, so
that the distinct bytes of a step (~830 MiB) exceed twice the 256 MiB
Infinity Cache and the kernel streams from HBM.  One step = segment build +
one fused BGMV launch over all 128 modules.  Inputs are resident in HBM
before timing starts.

Prints ONE JSON line.  `value` is tokens/s; `roofline` gives the BGMV
kernel's algorithmic bytes per launch over its average duration (HIP events
on the launch stream) against the 8 TB/s HBM peak; `cpu_baseline` is the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-apply tokens/s; achieved HBM GB/s (BGMV) and MFMA TFLOP/s (SGMV) vs peak"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bgmv_decode_x128",
                    choices=["bgmv_decode_x128", "bgmv_decode", "sgmv_prefill", "mixed_rank", "encoder_step"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def make_workload(name):
    import workloads as W
    if name == "bgmv_decode_x128":
        return W.c2_bgmv_decode(n_modules=128, draw_w=False), "bgmv", {
            "workload": "bgmv_decode_x128", "tokens": 64, "h_in": 4096, "h_out": 4096, "rank": 16,
            "slots": 32, "ids": "finite Zipf(1.1) over 32 slots", "modules_per_launch": 128}
    if name == "bgmv_decode":
        return W.c2_bgmv_decode(draw_w=False), "bgmv", {
            "workload": "bgmv_decode", "tokens": 64, "h_in": 4096, "h_out": 4096, "rank": 16, "slots": 32,
            "ids": "finite Zipf(1.1) over 32 slots", "modules_per_launch": 1}
    if name == "sgmv_prefill":
        return W.c3_sgmv_prefill(draw_w=False), "sgmv", {
            "workload": "sgmv_prefill", "tokens": 4096, "segments": 8, "h": 4096, "rank": 16,
            "modules": "q,k,v,o (q,k,v share x)"}
    if name == "mixed_rank":
        return W.c4_mixed_rank(draw_w=False), "sgmv", {
            "workload": "mixed_rank", "tokens": 1072, "ranks": "8/16/32/64", "slots": 64, "h": 4096}
    return W.c5_encoder_step(draw_w=False), "sgmv", {
        "workload": "encoder_step", "tokens": 32768, "slots": 1024, "rank": 16,
        "modules": "qkv 768->2304, o 768->768, up 768->3072, down 3072->768"}


def cpu_baseline(wl, seconds):
    """The oracle, untouched, on one core: whole steps (all modules, all tokens) until `seconds`."""
    from threadpoolctl import threadpool_limits
    from oracle import lora_oracle as lo
    steps, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            for m in range(wl.n_modules):
                lo.lora_delta(wl, m)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or (steps >= 1 and el * (steps + 1) / steps > 3 * seconds):
                break
    return {"value": wl.n_tokens * steps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole step(s): {wl.n_tokens} tokens x {wl.n_modules} modules, fp64 "
                      f"per-token loop, {el:.1f} s on one core (BLAS threads = 1)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see DESIGN.md, 'Sharding').",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from segmented_gathered_rank_amd import accounting
    from segmented_gathered_rank_amd.harness import DeviceWorkload

    wl, mode, config = make_workload(args.workload)
    dw = DeviceWorkload(wl, device=0)
    stream = torch.cuda.current_stream()
    work = accounting.step_work(wl, fused=(mode == "bgmv"))

    def step(ev=None):
        dw.build_segments()
        if ev is not None:
            ev[0].record(stream)
        if mode == "bgmv":
            dw.bgmv()
        else:
            dw.shrink()
            dw.expand()
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))

    extra = {"apply_ms_mean": kern_avg, "apply_ms_min": float(np.min(kern_ms)),
             "algorithmic_bytes_per_step": work["bytes"], "flops_per_step": work["flops"],
             "achieved_tflops": work["flops"] / (kern_avg * 1e-3) / 1e12}
    if mode == "bgmv" and wl.n_modules > 1:
        # one-module calls (the decode batch as the config states it), replayed from a
        # captured graph so that host launch cost is not in the figure
        import segmented_gathered_rank_amd as sgr
        y = dw.y[0]
        calls = 16
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                sgr.lora_apply_bgmv(dw.pool, i, 1, dw._xp(dw.x_off[i]), 4096, 0, dw.seg, y[i], 4096, 0,
                                    sgr.LORA_BF16)
        g.replay()
        torch.cuda.synchronize()
        lat = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            lat.append(a.elapsed_time(b) / calls)
        extra["single_module_call_us"] = float(np.median(lat) * 1e3)
        extra["single_module_bytes"] = work["per_module"][0]["bytes"]
        extra["single_module_GBps"] = work["per_module"][0]["bytes"] / (np.median(lat) * 1e-3) / 1e9

    bound_bytes = work["bytes"]
    achieved = bound_bytes / (kern_avg * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_bgmv" if mode == "bgmv" else "shrink+expand",
                "bytes_per_launch": bound_bytes}
    out = {
        "metric": METRIC, "value": round(wl.n_tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": config, "roofline": roofline, "extra": extra,
    }
    dw.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
