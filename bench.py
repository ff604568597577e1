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
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bgmv_decode_x128",
                    choices=["bgmv_decode_x128", "bgmv_decode", "sgmv_prefill", "mixed_rank", "encoder_step",
                             "encoder_fused", "prefill_fused", "encoder_fused_fp8", "prefill_fused_fp8",
                             "tiers_trace"])
    ap.add_argument("--path", choices=["auto", "bgmv", "sgmv"], default="auto",
                    help="force the fused BGMV or the shrink+expand path (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets the steps cycle through (each with its own pool, x and y); default: enough "
                         "that one cycle moves more than twice the 256 MB Infinity Cache")
    ap.add_argument("--no-single-module", action="store_true",
                    help="skip the one-module calls of the decode batch (timed by default, replayed from a graph)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the GPU apply times of the prefill, mixed-rank and encoder configs (default workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="copy a buffer of this size once before timing (reference for HBM counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) instead of benchmarking")
    ap.add_argument("--pmc-kernel", default="k_gemvILi0E", help="substring of the kernel to summarize")
    ap.add_argument("--pmc-out", default=None, help="write the traffic summary JSON here")
    ap.add_argument("--pmc-mfma-summary", metavar="DIR",
                    help="summarize a rocprofv3 --pmc run of the matrix-core counters (MFMA busy and ops, CU busy, "
                         "LDS bank conflicts) for the kernels named by --pmc-kernel (name substrings separated by semicolons)")
    ap.add_argument("--pmc-per-step", type=int, default=0,
                    help="the step makes this many launches of the kernel (one per module): average over all "
                         "of them and report HBM bytes per step")
    return ap.parse_args()


# Input sets per workload.  One set of the 128-module decode batch moves 0.87 GB per
# step, yet back-to-back launches over it ran 17% faster than over two alternating
# sets (three sets: the same as two): the Infinity Cache still held part of it.
ROTATE = {"bgmv_decode_x128": 2, "sgmv_prefill": 2, "mixed_rank": 16}


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
    if name == "encoder_fused":
        return W.c5_encoder_step(), "fused", {
            "workload": "encoder_fused", "tokens": 32768, "slots": 1024, "rank": 16,
            "modules": "qkv 768->2304, o 768->768, up 768->3072, down 3072->768",
            "step": "y = x W + adapter term per module, one lora_fused_gemm call each"}
    if name in ("encoder_fused_fp8", "prefill_fused_fp8"):
        base = W.c5_encoder_step() if name == "encoder_fused_fp8" else W.c3_sgmv_prefill()
        return W.with_fp8_base(base), "fused8", {
            "workload": name, "tokens": base.n_tokens, "rank": 16,
            "modules": ("qkv 768->2304, o 768->768, up 768->3072, down 3072->768" if name == "encoder_fused_fp8"
                        else "q,k,v,o 4096->4096 (q,k,v share x)"),
            "base": "W as OCP FP8 E4M3 with one float32 scale per output column; x, adapters, y bf16",
            "step": "y = x W + adapter term per module, one lora_fused_gemm_fp8w call each"}
    if name == "prefill_fused":
        return W.c3_sgmv_prefill(), "fused", {
            "workload": "prefill_fused", "tokens": 4096, "segments": 8, "h": 4096, "rank": 16,
            "modules": "q,k,v,o (q,k,v share x)",
            "step": "y = x W + adapter term per module, one lora_fused_gemm call each"}
    return W.c5_encoder_step(draw_w=False), "sgmv", {
        "workload": "encoder_step", "tokens": 32768, "slots": 1024, "rank": 16,
        "modules": "qkv 768->2304, o 768->768, up 768->3072, down 3072->768"}


# HIP sources that build the kernel whose HBM traffic a workload's counters measured, and
# its launch (apply.hip sizes the grids): a change to any of them voids the stored counters.
KERNEL_SOURCES = {
    "bgmv_decode_x128": ["common.hpp", "segments_wave.hpp", "gemv_kernels.hpp", "apply.hip"],
    "encoder_fused": ["common.hpp", "fused_gemm.hpp", "apply.hip"],
    "prefill_fused": ["common.hpp", "fused_gemm.hpp", "apply.hip"],
}
ALL_KERNEL_SOURCES = ["common.hpp", "segments_wave.hpp", "gemv_kernels.hpp", "mfma_kernels.hpp", "fused_gemm.hpp",
                      "apply.hip", "segments.hip"]


def kernel_source_sha(workload):
    """sha256 over the HIP sources of the workload's measured kernel (identifies its version)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(workload, ALL_KERNEL_SOURCES):
        with open(os.path.join(ROOT, "segmented_gathered_rank_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload):
    """Counter-measured HBM bytes per launch, if taken on the current kernel sources."""
    try:
        with open(traffic_file(workload)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha(workload):
        return None
    return t.get("hbm_bytes_per_step", t.get("hbm_bytes_per_launch"))


def pmc_summary(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the target kernel, each scaled by what the
    same counter reads for the calibration copy of known size in the same run."""
    import csv
    import glob

    def rows(d):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    res = {}
    for name, d in (("FETCH_SIZE", args.pmc_summary[0]), ("WRITE_SIZE", args.pmc_summary[1])):
        rs = [r for r in rows(d) if r["Counter_Name"] == name]
        copies = [float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]]
        match = [r for r in rs if args.pmc_kernel in r["Kernel_Name"]]
        big = max((int(r["Grid_Size"]) for r in match), default=0)     # the bench's own launch shape
        target = [float(r["Counter_Value"]) for r in match
                  if args.pmc_per_step > 0 or int(r["Grid_Size"]) == big]
        if not copies or not target:
            raise SystemExit(f"{name}: no copy or no target dispatch found in {d}")
        ref_kib = args.calibrate_copy_mib * 1024.0
        res[name] = {"kernel_kib_mean": sum(target) / len(target), "dispatches": len(target),
                     "grid_size": big, "copy_kib": max(copies), "copy_expected_kib": ref_kib,
                     "scale": ref_kib / max(copies)}
    hbm = 1024.0 * (res["FETCH_SIZE"]["kernel_kib_mean"] * res["FETCH_SIZE"]["scale"] +
                    res["WRITE_SIZE"]["kernel_kib_mean"] * res["WRITE_SIZE"]["scale"])
    out = {"workload": args.workload, "kernel": args.pmc_kernel, "kernel_source_sha": kernel_source_sha(args.workload),
           "hbm_bytes_per_launch": hbm, "counters": res}
    if args.pmc_per_step > 0:   # every launch of the step, averaged, times the launches per step
        out["hbm_bytes_per_step"] = hbm * args.pmc_per_step
        out["launches_per_step"] = args.pmc_per_step
    if args.pmc_out:
        with open(args.pmc_out, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps(out))


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]


def pmc_mfma_summary(args):
    """Per kernel (name substrings of --pmc-kernel), each counter averaged over its
    dispatches, and: MFMA utilisation = MFMA busy cycles over (GPU active cycles x
    SIMDs), the rocprofv3 MfmaUtil expression, with GRBM_GUI_ACTIVE summed over the
    8 XCDs divided by 8 and 1,024 SIMDs (256 CUs x 4); bf16 MFMA flops = MOPS x 512
    (per dispatch);
    LDS bank-conflict cycles per LDS-active cycle (SQ_ACTIVE_INST_LDS is in quad-cycles)."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(args.pmc_mfma_summary, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    out = {}
    for pat in args.pmc_kernel.split(";"):
        disp = {}
        for r in rows:
            if pat in r["Kernel_Name"]:
                disp.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        full = [d for d in disp.values() if all(c in d for c in MFMA_COUNTERS)]
        if not full:
            raise SystemExit(f"no dispatch of {pat!r} with all counters in {args.pmc_mfma_summary}")
        avg = {c: sum(d[c] for d in full) / len(full) for c in MFMA_COUNTERS}
        active = avg["GRBM_GUI_ACTIVE"] / 8.0
        out[pat] = {"dispatches": len(full), "counters_mean": avg,
                    "mfma_util_pct": round(100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * 1024), 2),
                    "bf16_mfma_flops": avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
                    "lds_bank_conflict_per_lds_cycle": round(avg["SQ_LDS_BANK_CONFLICT"] /
                                                             max(4 * avg["SQ_ACTIVE_INST_LDS"], 1.0), 4)}
    print(json.dumps(out, indent=1))


def copy_gbps(mib=1024, reps=10):
    """Measured device-to-device copy bandwidth (read + write bytes per second):
    the streaming rate this GPU reaches, a second denominator beside the spec peak."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def base_gemm_ms(wl, reps=10):
    """The shared base products y0 = x W of every module (bf16, hipBLASLt through
    torch.matmul into preallocated outputs) on random data of the workload's
    shapes, the faster of the two weight layouts: the denominator of the
    adapter overhead.  Not part of the library or of the timed step."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    flops = sum(2.0 * wl.n_tokens * m.h_in * m.h_out for m in wl.modules)
    best = None
    for transposed in (False, True):   # W stored [h_in][h_out], or as a linear layer's [h_out][h_in]
        ops = []
        for m in wl.modules:
            x = torch.randn(wl.n_tokens, m.h_in, device="cuda", dtype=torch.bfloat16, generator=g)
            if transposed:
                w = torch.randn(m.h_out, m.h_in, device="cuda", dtype=torch.bfloat16, generator=g).t()
            else:
                w = torch.randn(m.h_in, m.h_out, device="cuda", dtype=torch.bfloat16, generator=g)
            ops.append((x, w, torch.empty(wl.n_tokens, m.h_out, device="cuda", dtype=torch.bfloat16)))
        for x, w, y in ops:
            torch.matmul(x, w, out=y)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for x, w, y in ops:
                torch.matmul(x, w, out=y)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        best = ms if best is None else min(best, ms)
        del ops
    return best, flops


_CPU_WL = None   # the workload the forked CPU workers read (set before their pool starts)


def _cpu_cores():
    """Host cores for the all-cores leg: the process's CPU set, at most 16 (a GPU machine's share per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_tokens(job):
    """The oracle on tokens [t0, t1) of modules [m0, m1) of _CPU_WL, BLAS threads = 1:
    the adapter term, or (fused) x W plus the term.  Returns token-modules done."""
    t0, t1, m0, m1, fused, fp8 = job
    from threadpoolctl import threadpool_limits
    from oracle import lora_oracle as lo
    wl = _CPU_WL
    f = (lo.lora_forward_fp8w if fp8 else lo.lora_forward) if fused else lo.lora_delta
    with threadpool_limits(1):
        for m in range(m0, m1):
            f(wl, m, range(t0, t1))
    return (t1 - t0) * (m1 - m0)


def cpu_baseline(wl, seconds, fused=False, fp8=False, block=64, base_wl=None):
    """The oracle as it stands, on the host's cores, over blocks of `block`
    tokens (every module) of the workload, in order, for about `seconds` per
    leg: one core, then all cores (forked workers, each a contiguous share of a
    block).  Runs before anything touches the GPU (the workers are forked).
    base_wl: a one-module workload with W drawn, whose fp64 base product x W is
    timed on one core as well (the base is not part of the adapter term)."""
    global _CPU_WL
    import multiprocessing
    _CPU_WL = wl
    n, nm = wl.n_tokens, wl.n_modules
    blocks = [(t, min(n, t + block)) for t in range(0, n, block)]
    # one core
    done, b, t0 = 0, 0, time.perf_counter()
    while True:
        done += _oracle_tokens((*blocks[b % len(blocks)], 0, nm, fused, fp8))
        b += 1
        el = time.perf_counter() - t0
        if el >= seconds or el * (b + 1) / b > 3 * seconds:
            break
    one = done / nm / el
    one_sample = f"{b} block(s) of up to {block} tokens x {nm} modules in {el:.1f} s"
    # all cores: a block's modules split over the workers when there are enough, else its tokens
    cores = _cpu_cores()
    jobs_of = []
    for (s0, s1) in blocks:
        if nm >= cores:
            cuts = [nm * k // cores for k in range(cores + 1)]
            jobs_of.append([(s0, s1, cuts[k], cuts[k + 1], fused, fp8) for k in range(cores) if cuts[k + 1] > cuts[k]])
        else:
            cuts = [s0 + (s1 - s0) * k // cores for k in range(cores + 1)]
            jobs_of.append([(cuts[k], cuts[k + 1], 0, nm, fused, fp8) for k in range(cores) if cuts[k + 1] > cuts[k]])
    split = "modules" if nm >= cores else "tokens"
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_tokens, jobs_of[0])            # workers up (not timed)
        done, b, t0 = 0, 0, time.perf_counter()
        while True:
            done += sum(pool.map(_oracle_tokens, jobs_of[b % len(jobs_of)]))
            b += 1
            el = time.perf_counter() - t0
            if el >= seconds or el * (b + 1) / b > 3 * seconds:
                break
    allc = done / nm / el
    out = {"value": round(one, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{one_sample}; fp64 per-token {'x W + adapter term' if fused else 'adapter term'} "
                     f"({'FP8 base, ' if fp8 else ''}the oracle as written), BLAS threads = 1",
           "all_cores": {"value": round(allc, 2), "unit": "tokens/s", "cores": cores,
                         "sample": f"{b} block(s) of up to {block} tokens, each block's {split} split over "
                                   f"{cores} forked workers, {el:.1f} s"},
           "cpu_model": _cpu_model()}
    if base_wl is not None:   # the shared base product x W of one module, fp64, one core
        from threadpoolctl import threadpool_limits
        from oracle import lora_oracle as lo
        with threadpool_limits(1):
            t0 = time.perf_counter()
            lo.base_product(base_wl, 0)
            el = time.perf_counter() - t0
        mod = base_wl.modules[0]
        out["base_product_fp64"] = {
            "seconds_per_module": round(el, 4), "tokens_per_s_per_module": round(base_wl.n_tokens / el, 2),
            "shape": f"{base_wl.n_tokens} tokens x {mod.h_in} -> {mod.h_out}, one core, row by row"}
    return out


def fused_work(wl, w_elem_bytes=2):
    """Algorithmic flops and bytes of one fused step: every module's base
    product (x read, W read, y written once) plus its adapter term (each
    distinct adapter's A and B pages read once).  w_elem_bytes 1: W as FP8
    codes plus one float32 scale per output column."""
    import numpy as np
    flops = byts = 0
    used = sorted(set(int(i) for i in np.unique(wl.ids) if 0 <= i < wl.n_slots))
    for m, mod in enumerate(wl.modules):
        n = wl.n_tokens
        flops += 2.0 * n * mod.h_in * mod.h_out
        byts += 2 * (n * mod.h_in + n * mod.h_out) + w_elem_bytes * mod.h_in * mod.h_out
        if w_elem_bytes == 1:
            byts += 4 * mod.h_out
        for i in range(n):
            a = wl.adapters[int(wl.ids[i])][m] if 0 <= wl.ids[i] < wl.n_slots else None
            if a is not None:
                flops += 2.0 * a[0] * (mod.h_in + mod.h_out)
        for s in used:
            a = wl.adapters[s][m]
            if a is not None:
                byts += 2 * a[0] * (mod.h_in + mod.h_out)
    return flops, byts


def time_ms(fn, reps=10):
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def tiers_trace(args):
    """The study page's request trace (500 rank-16 adapters of 4096 x 4096,
    Zipf(1.1), 50,000 requests, LCG seed 11) served in decode batches of 32
    requests through 32 GPU slots and a 500-adapter host tier: per batch one
    lora_tiers_acquire (uploads of GPU misses from page-locked host memory,
    cold loads from numpy arrays through the fetch callback), a segment build
    and one fused BGMV; the host never waits for the GPU inside the loop.
    Against the same loop with all 500 adapters resident in a 500-slot pool,
    and with a forecast: after each batch the next batch's adapters are
    prefetched on a copy stream.  Wall clock over the whole trace, host work
    included."""
    import numpy as np
    import torch
    import segmented_gathered_rank_amd as sgr
    import workloads as W
    from workloads import _store, _normal
    n_ad, gpu_slots, host_slots, bsz, h, r = 500, 32, 500, 32, 4096, 16
    trace = W.request_trace()
    rng = np.random.default_rng(7)
    A = [_store(_normal(rng, 0.02, (r, h)), "bf16") for _ in range(n_ad)]
    B = [_store(_normal(rng, 0.02, (r, h)), "bf16") for _ in range(n_ad)]
    dev = torch.device("cuda", 0)
    x = torch.randn(bsz, h, device=dev).to(torch.bfloat16)
    y = torch.zeros(bsz, h, device=dev, dtype=torch.bfloat16)

    def run(tiered, prefetch=False):
        slots = gpu_slots if tiered else n_ad
        pool = sgr.lora_pool_create(0, sgr.LORA_BF16, h, slots * 2 * r, slots, 1, [h], [h], r)
        seg_buf = torch.zeros(max(sgr.lora_segments_bytes(bsz, slots), 256), dtype=torch.uint8, device=dev)
        seg = sgr.lora_segments_bind(seg_buf, bsz, slots)
        tiers = sgr.lora_tiers_create(gpu_slots, host_slots) if tiered else None
        if not tiered:
            for a in range(n_ad):
                sgr.lora_pool_load(pool, a, 0, r, A[a], B[a], 2.0)
        fetch = lambda a, m: (r, 2.0, A[a], B[a])
        copy = torch.cuda.Stream() if prefetch else None
        # the batch's slot ids reach the device through a ring of page-locked buffers without
        # blocking the host (an entry is rewritten only after its copy has run)
        ring = 4
        h_ids = [torch.empty(bsz, dtype=torch.int32, pin_memory=True) for _ in range(ring)]
        d_ring = [torch.empty(bsz, dtype=torch.int32, device=dev) for _ in range(ring)]
        copied = [None] * ring
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k, b0 in enumerate(range(0, len(trace), bsz)):
            req = trace[b0:b0 + bsz]
            ids = sgr.lora_tiers_acquire(tiers, pool, req, fetch) if tiered else req
            j = k % ring
            if copied[j] is not None:
                copied[j].synchronize()
            h_ids[j].numpy()[:len(ids)] = np.asarray(ids, dtype=np.int32)
            d_ids = d_ring[j][:len(ids)]
            d_ids.copy_(h_ids[j][:len(ids)], non_blocking=True)
            copied[j] = torch.cuda.Event()
            copied[j].record()
            sgr.lora_build_segments(d_ids, seg)
            sgr.lora_apply_bgmv(pool, 0, 1, x, h, 0, seg, y, h, 0, sgr.LORA_BF16)
            if prefetch:   # the forecast: the next batch of the queue
                sgr.lora_tiers_batch_done(tiers)
                sgr.lora_tiers_prefetch(tiers, pool, trace[b0 + bsz:b0 + 2 * bsz], fetch, copy)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = sgr.lora_tiers_stats(tiers) if tiered else None
        if tiered:
            sgr.lora_tiers_destroy(tiers)
        sgr.lora_pool_destroy(pool)
        return wall, st

    run(True)   # warm-up of both paths (library, allocator, page-locked buffers)
    run(False)
    t_res, _ = run(False)
    t_tier, st = run(True)
    t_pf, st_pf = run(True, prefetch=True)
    n = len(trace)
    misses = st["host_hits"] + st["cold_loads"]
    adapter_bytes = 2 * r * 2 * h
    out = {
        "metric": METRIC, "value": round(n / t_tier, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": n // bsz, "warmup": 0, "ms_per_step": round(t_tier * 1e3 / (n // bsz), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "tiers_trace", "adapters": n_ad, "gpu_slots": gpu_slots, "host_slots": host_slots,
                   "requests": n, "batch": bsz, "h": h, "rank": r, "ids": "the study page's LCG trace, Zipf(1.1)"},
        "roofline": None,
        "extra": {"gpu_hit_pct": round(100.0 * st["gpu_hits"] / n, 1),
                  "host_hit_pct": round(100.0 * st["host_hits"] / n, 1), "cold_loads": st["cold_loads"],
                  "resident_tokens_per_s": round(n / t_res, 1), "tiered_over_resident_time": round(t_tier / t_res, 3),
                  "upload_us_per_miss": round((t_tier - t_res) / max(misses, 1) * 1e6, 2),
                  "upload_GBps_per_miss": round(adapter_bytes * misses / max(t_tier - t_res, 1e-9) / 1e9, 2),
                  "prefetch_tokens_per_s": round(n / t_pf, 1),
                  "prefetch_gpu_hit_pct": round(100.0 * st_pf["gpu_hits"] / n, 1),
                  "prefetch_host_hit_pct": round(100.0 * st_pf["host_hits"] / n, 1),
                  "prefetch_cold_loads": st_pf["cold_loads"],
                  "note": "wall clock of the serve loop, host work included; upload cost = extra time over the "
                          "resident loop per GPU miss"},
    }
    print(json.dumps(out), flush=True)


def sgmv_calls_of(dw):
    """The library calls the harness's apply() makes for a workload."""
    if not dw.sgmv_fused_calls():
        return "lora_shrink + lora_expand"
    return "lora_apply_sgmv" if len(dw._x_runs(*dw.groups[0])) == 1 else "lora_apply_sgmv_multi"


def config_runs(DeviceWorkload, accounting, steps=20, warmup=3):
    """GPU apply time (the adapter term through the harness's calls: lora_apply_sgmv
    where one call covers the step, else lora_shrink + lora_expand; HIP events on the
    launch stream) and
    step time (segment build + apply) of the prefill, mixed-rank and encoder
    configs, each cycling through its input sets; HBM fraction of the apply
    from its algorithmic bytes."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    res = {}
    for name in ("sgmv_prefill", "mixed_rank", "encoder_step"):
        wl, _, _ = make_workload(name)
        sets = ROTATE.get(name, 1)
        dws = [DeviceWorkload(wl, device=0) for _ in range(sets)]
        work = accounting.step_work(wl, fused=False)
        for i in range(warmup):
            d = dws[i % sets]
            d.build_segments()
            d.apply()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            d = dws[i % sets]
            ev[i][0].record(stream)
            d.build_segments()
            ev[i][1].record(stream)
            d.apply()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        apply = np.array([e[1].elapsed_time(e[2]) for e in ev])
        stepm = np.array([e[0].elapsed_time(e[2]) for e in ev])
        gbps = work["bytes"] / (apply.mean() * 1e-3) / 1e9
        res[name] = {"apply_ms_mean": round(float(apply.mean()), 5), "apply_ms_min": round(float(apply.min()), 5),
                     "step_ms_mean": round(float(stepm.mean()), 5), "tokens": wl.n_tokens,
                     "tokens_per_s": round(wl.n_tokens / (stepm.mean() * 1e-3), 1),
                     "algorithmic_bytes": work["bytes"], "hbm_GBps": round(gbps, 1),
                     "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4), "input_sets": sets,
                     "calls": sgmv_calls_of(dws[0])}
        for d in dws:
            d.close()
        del dws
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.pmc_mfma_summary:
        pmc_mfma_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (tokens shard across data-parallel "
              "replicas with no exchange; tensor-parallel row splits would add one all-reduce of t).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "tiers_trace":
        tiers_trace(args)
        return
    wl, mode, config = make_workload(args.workload)
    if args.path != "auto":
        mode = args.path
        config["path"] = mode
    cpu = None
    if not args.no_cpu_baseline:   # first: the all-cores leg forks workers, before the GPU is touched
        import workloads as W
        base_wl = W.c2_bgmv_decode(seed=12, n_modules=1) if mode == "bgmv" else None
        cpu = cpu_baseline(wl, args.cpu_seconds, fused=mode in ("fused", "fused8"), fp8=mode == "fused8",
                           base_wl=base_wl)
    import numpy as np
    import torch
    from segmented_gathered_rank_amd import accounting
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    # input sets the steps cycle through, so that a cycle's distinct bytes exceed twice the
    # 256 MB Infinity Cache and the kernels read from HBM: the decode batch covers that with its
    # 128 modules in one launch, the prefill step (346 MB) takes 2 sets, the mixed batch (43 MB) 16
    rotate = args.rotate if args.rotate > 0 else ROTATE.get(args.workload, 1)
    dws = [DeviceWorkload(wl, device=0) for _ in range(rotate)]
    dw = dws[0]
    config["input_sets"] = rotate
    stream = torch.cuda.current_stream()
    work = accounting.step_work(wl, fused=(mode == "bgmv"))

    if mode == "fused":
        for d in dws:
            d.upload_weights()
    if mode == "fused8":
        for d in dws:
            d.upload_weights_fp8()
            d.upload_weights()   # the bf16 pass of the same layer, timed beside it

    # a decode batch of at most 64 tokens runs straight from its ids (lora_apply_bgmv_ids): each
    # workgroup of the one launch builds the batch's unit list itself, so the step has no
    # separate segment build
    ids_path = mode == "bgmv" and wl.n_tokens <= 64

    def step(ev=None, i=0):
        d = dws[i % rotate]
        if mode not in ("fused", "fused8") and not ids_path:
            d.build_segments()
        if ev is not None:
            ev[0].record(stream)
        if mode == "bgmv":
            if ids_path:
                d.bgmv_ids()
            else:
                d.bgmv()
        elif mode == "fused":
            d.fused()
        elif mode == "fused8":
            d.fused_fp8()
        else:
            d.apply()     # lora_apply_sgmv where one call covers the step, else shrink + expand calls
        if ev is not None:
            ev[1].record(stream)

    if args.calibrate_copy_mib > 0:   # a plain device copy of known size, for the HBM counters
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the GPU's clocks settle only after some milliseconds of steady work (the first few dozen
    # steps of a cold box ran about 6% slower): untimed steps for about 100 ms, then the
    # warm-up steps proper
    t_warm = time.perf_counter()
    for i in range(2000):
        step(None, i)
        if i % 8 == 7:
            torch.cuda.synchronize()
            if time.perf_counter() - t_warm > 0.1:
                break
    for i in range(args.warmup):
        step(None, i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    ms_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))

    extra = {"apply_ms_mean": kern_avg, "apply_ms_min": float(np.min(kern_ms)),
             "algorithmic_bytes_per_step": work["bytes"], "flops_per_step": work["flops"],
             "achieved_tflops": work["flops"] / (kern_avg * 1e-3) / 1e12}
    if mode == "bgmv" and wl.n_modules > 1 and not args.no_single_module:
        # one-module calls (the decode batch as the config states it), replayed from a
        # captured graph so that host launch cost is not in the figure
        import segmented_gathered_rank_amd as sgr
        dw.build_segments()   # the ids path of the step does not build them
        torch.cuda.synchronize()
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
    if ids_path:
        # the same step through the segment builder: lora_build_segments + lora_apply_bgmv, two launches
        k = [0]

        def segments_step():
            d = dws[k[0] % rotate]
            k[0] += 1
            d.build_segments()
            d.bgmv()
        extra["segments_path_step_ms"] = round(time_ms(segments_step, reps=20), 5)

    if mode in ("fused", "fused8"):
        fp8 = mode == "fused8"
        flops, byts = fused_work(wl, 1 if fp8 else 2)
        tf = flops / (kern_avg * 1e-3) / 1e12
        base_ours = time_ms(lambda: (dw.fused_fp8 if fp8 else dw.fused)(adapters=False))
        gms, _ = base_gemm_ms(wl)
        unfused = time_ms(lambda: dw.sgmv_step())
        extra = {"fused_ms_mean": kern_avg, "fused_ms_min": float(np.min(kern_ms)), "flops_per_step": flops,
                 "algorithmic_bytes_per_step": byts, "arith_intensity_flop_per_byte": round(flops / byts, 1),
                 "base_only_ms": round(base_ours, 4), "adapter_overhead_in_kernel": round(kern_avg / base_ours - 1, 4),
                 "hipblaslt_base_ms": round(gms, 4), "unfused_lora_step_ms": round(unfused, 4),
                 "hipblaslt_plus_unfused_ms": round(gms + unfused, 4),
                 "fused_over_hipblaslt_plus_unfused": round(kern_avg / (gms + unfused), 4),
                 "fused_over_hipblaslt_base": round(kern_avg / gms, 4)}
        if fp8:   # the bf16 pass of the same layer and its W bytes, beside the FP8 one
            bf16_ms = time_ms(lambda: dw.fused())
            _, byts16 = fused_work(wl, 2)
            extra.update({"bf16_fused_ms": round(bf16_ms, 4), "fp8_over_bf16_fused": round(kern_avg / bf16_ms, 4),
                          "w_bytes_fp8": int(sum(m.h_in * m.h_out + 4 * m.h_out for m in wl.modules)),
                          "w_bytes_bf16": int(sum(2 * m.h_in * m.h_out for m in wl.modules)),
                          "algorithmic_bytes_bf16_pass": byts16})
        # traffic: counter-measured HBM bytes of one step (all its launches), against
        # algorithmic_bytes_per_step
        roofline = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(args.workload),
                    "kernel": "k_fused_gemm<W8>" if fp8 else "k_fused_gemm", "flops_per_launch_set": flops}
        out = {
            "metric": METRIC, "value": round(wl.n_tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": config, "roofline": roofline, "extra": extra,
        }
        for d in dws:
            d.close()
        if cpu is not None:
            out["cpu_baseline"] = cpu
        print(json.dumps(out), flush=True)
        return

    bound_bytes = work["bytes"]
    achieved = bound_bytes / (kern_avg * 1e-3) / 1e9
    if args.calibrate_copy_mib <= 0:   # in counter runs the calibration copy must stay the largest copy
        extra["copy_GBps"] = round(copy_gbps(), 1)
        extra["frac_of_copy_GBps"] = round(achieved / extra["copy_GBps"], 4)
    if mode == "sgmv":   # the matrix-core path: what its arithmetic intensity allows at the HBM peak
        ai = work["flops"] / work["bytes"]
        attainable = min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
        extra["mfma_peak_tflops"] = MFMA_BF16_PEAK_TFLOPS
        extra["arith_intensity_flop_per_byte"] = round(ai, 2)
        extra["attainable_tflops"] = round(attainable, 2)
        extra["frac_of_peak_tflops"] = round(extra["achieved_tflops"] / MFMA_BF16_PEAK_TFLOPS, 5)
        extra["frac_of_attainable_tflops"] = round(extra["achieved_tflops"] / attainable, 4)
    if args.workload == "encoder_step":
        gms, gflops = base_gemm_ms(wl)
        extra["base_gemm_ms"] = round(gms, 4)
        extra["base_gemm_tflops"] = round(gflops / (gms * 1e-3) / 1e12, 1)
        extra["lora_apply_over_base_gemm"] = round(kern_avg / gms, 4)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(args.workload),
                "kernel": ("k_bgmv_ids (fused BGMV from the ids)" if ids_path else "k_gemv<0> (fused BGMV)")
                if mode == "bgmv" else "shrink+expand",
                "bytes_per_launch": bound_bytes}
    out = {
        "metric": METRIC, "value": round(wl.n_tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": config, "roofline": roofline, "extra": extra,
    }
    for d in dws:
        d.close()
    del dws, dw
    torch.cuda.empty_cache()
    if args.workload == "bgmv_decode_x128" and not args.no_configs:
        extra["configs"] = config_runs(DeviceWorkload, accounting)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
