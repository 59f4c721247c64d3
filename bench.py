"""Benchmark: fused Hadamard-quantize + W4A4/W4A8 GEMM throughput on
CogVideoX-5B-shaped DiT block linears (one MI355X).

One step = one pass of the whole hot path over one block:
  for each linear (QKV 3072->9216, out 3072->3072, FFN-up 3072->12288,
  FFN-down 12288->3072) at M = 17776 tokens:
      hadamard_quantize (NVFP4 with the tensor amax computed, or INT8)
      + qgemm_w4a4 / qgemm_w4a8 (bf16 output)
  block_stats over the block input/output and the cached delta, the 8
  statistics copied to pinned host memory, and dmpq_step for the block on
  them (on the host, overlapping the next step's GPU work, as in a model
  with more than one block).
The headline step uses the 50/50 NVFP4/INT8 assignment (QKV and FFN-down
NVFP4, out-proj and FFN-up INT8), the W4A6 operating point of the pages; the
same point with the two formats swapped, the all-NVFP4, all-INT8 and
all-W4A16 sweeps are timed the same way after it,
then the MX-native variant (MXFP4 weights; MXFP4 / MXFP8 activations on the
block-scaled MFMA) with the same 50/50 assignment, all-MXFP4 and all-MXFP8.

value = sum of 2*M*N*K over the four linears / step time (TOPS).  Inputs are
seeded synthetic bf16 (Laplace(0,1) with 0.5% of the channels x30), resident
in HBM before the timed region; weights are random N(0, 0.02) prepared
offline (Hadamard-rotated + NVFP4) before timing.  The timed steps record
no events inside them; the per-call times and the per-step spread come from
a second pass of the same steps with HIP events around every call.

Besides the step, the JSON line carries: the dominant GEMM call against the
fp16 MFMA peak (roofline, with counter traffic while the committed record
matches the sources), each quantize pass against HBM peak and against a
plain streaming pass of the same bytes and launch size, the MX GEMMs
against their own peaks, block_stats against HBM peak, the same four GEMMs
in bf16 through torch / hipBLASLt (context), the 1080p FFN stress shape,
the fused FFN-up -> FFN-down epilogue, the closed-loop schedule study, the
host cost of dmpq_step, and the CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--no-cpu-baseline]
                       [--no-dyn] [--no-stress] [--sweeps a,b,...]
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_FP16_MFMA_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_INT8_TOPS = 5000.0
HAD_BLOCK = 64

MIXED = {"qkv": "nvfp4", "out": "int8", "ffn_up": "int8", "ffn_down": "nvfp4"}
SWEEPS = {"mixed_w4a6": MIXED,
          # the same 50/50 point with the two formats swapped between the linears
          "mixed_w4a6_swapped": {k: ("int8" if v == "nvfp4" else "nvfp4") for k, v in MIXED.items()},
          "all_w4a4": {k: "nvfp4" for k in MIXED},
          "all_w4a8": {k: "int8" for k in MIXED},
          # the full-precision fallback (bf16 activations, 4-bit weights) on every linear
          "all_w4a16": {k: "bf16" for k in MIXED},
          # the MX-native variant: MXFP4 weights, MXFP4 / MXFP8 activations on the
          # block-scaled MFMA, same 50/50 assignment, then all-4-bit / all-8-bit
          "mx_mixed": {k: ("mxfp4" if v == "nvfp4" else "mxfp8") for k, v in MIXED.items()},
          "all_mxfp4": {k: "mxfp4" for k in MIXED},
          "all_mxfp8": {k: "mxfp8" for k in MIXED}}
GEMM_OF = {"nvfp4": "qgemm_w4a4", "int8": "qgemm_w4a8", "bf16": "qgemm_w4a16", "mxfp4": "qgemm_mx",
           "mxfp8": "qgemm_mx"}
MX_PEAK = {"mxfp4": PEAK_FP4_TFLOPS, "mxfp8": PEAK_FP8_TFLOPS}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-dyn", action="store_true", help="skip the closed-loop schedule measurement")
    ap.add_argument("--no-stress", action="store_true", help="skip the 1080p FFN measurement")
    ap.add_argument("--sweeps", default=",".join(SWEEPS),
                    help="comma-separated subset of " + ",".join(SWEEPS) + " (the first listed is the headline)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run one plain elementwise pass over 512 MiB (reads 512 MiB, "
                         "writes 512 MiB): the reference for counter runs")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path runs on a single MI355X "
              "(the multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import video_diffusion_transformer_block_amd as V

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M = synth.TOKENS_2B_5B
    hidden = 3072
    linears = synth.block_linears(hidden)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    chosen = [w for w in args.sweeps.split(",") if w]
    want_mx = any(f.startswith("mx") for sw in chosen for f in SWEEPS[sw].values())
    X, W, WM, host = {}, {}, {}, {}
    for name, K, N in linears:
        x, w = synth.layer_inputs(M, name, K, N)
        host[name] = (x, w)
        X[name], W[name] = up(x), V.hadamard_quantize(up(w), HAD_BLOCK, "nvfp4")  # offline weight prep
        if want_mx:
            WM[name] = V.hadamard_quantize(up(w), HAD_BLOCK, "mxfp4")
    # the block's input: in the model the QKV linear reads LayerNorm(block
    # input), another tensor, so block_stats reads a buffer of its own and
    # does not warm the caches for the next step's QKV quantize
    Xblk = X["qkv"].clone()
    dprev = torch.zeros((M, hidden), dtype=torch.bfloat16, device=dev)
    dnew = torch.empty_like(dprev)
    Y = {name: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for name, K, N in linears}
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    flops = {name: 2.0 * M * N * K for name, K, N in linears}
    total_flops = sum(flops.values())
    params, state = V.dmpq_params(), V.dmpq_state()
    pinned = [torch.empty(8, dtype=torch.float64, pin_memory=True) for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    sched = {"count": 0, "pending": None}

    def step(assign, rec=None):
        nonlocal dprev, dnew
        for name, K, N in linears:
            fmt = assign[name]
            if rec is not None:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record()
            a = V.hadamard_quantize(X[name], HAD_BLOCK, fmt, stats=(name == "qkv"))
            if rec is not None:
                e1.record()
            if fmt == "nvfp4":
                V.qgemm_w4a4(a, W[name], None, "bf16", y=Y[name])
            elif fmt == "int8":
                V.qgemm_w4a8(a, W[name], None, "bf16", y=Y[name])
            elif fmt == "bf16":
                V.qgemm_w4a16(a, W[name], None, "bf16", y=Y[name])
            else:
                V.qgemm_mx(a, WM[name], None, "bf16", y=Y[name])
            if rec is not None:
                e2.record()
                rec.append((name, fmt, e0, e1, e2))
        _, st = V.block_stats(Xblk, Y["ffn_down"], dprev, dnew)
        # The 8 statistics go to pinned host memory without blocking; the host
        # scheduler runs on them while the GPU works on the next step, as it
        # does when a model has more than one block.
        slot = sched["count"] % 2
        sched["count"] += 1
        pinned[slot].copy_(st, non_blocking=True)
        copied[slot].record()
        if sched["pending"] is not None:
            consume(sched["pending"])
        sched["pending"] = slot
        dprev, dnew = dnew, dprev

    def consume(slot):
        copied[slot].synchronize()
        s = pinned[slot].numpy()
        ratio = V.outlier_ratio(s[4], s[5], M * hidden)
        V.dmpq_step(params, state, s, ratio)

    def drain():
        if sched["pending"] is not None:
            consume(sched["pending"])
            sched["pending"] = None

    results = {}
    for sweep in chosen:
        assign = SWEEPS[sweep]
        for _ in range(args.warmup):
            step(assign)
        drain()
        torch.cuda.synchronize()
        # no Python garbage collection inside the timed region: a collection
        # pause on the host would leave the GPU idle between launches
        gc.collect()
        gc.disable()
        # the breakdown pass: K steps with HIP events around every quantize
        # and GEMM call.  Each event record leaves the GPU idle for a few us
        # (about 65 us per step in all), so these steps run slower than the
        # timed ones; the per-call times (which include one such gap each)
        # and the per-step spread come from them.  It runs first: the GPU
        # takes some tens of ms of this load to reach its steady clock.
        rec = []
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb0.record()
        for _ in range(args.steps):
            step(assign, rec)
        eb1.record()
        drain()
        torch.cuda.synchronize()
        ms_instr = eb0.elapsed_time(eb1) / args.steps
        # the timed region: K whole steps with nothing recorded inside them
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tw = time.perf_counter()
        ev0.record()
        for _ in range(args.steps):
            step(assign)
        ev1.record()
        drain()
        torch.cuda.synchronize()
        wall = time.perf_counter() - tw
        gc.enable()
        ms = ev0.elapsed_time(ev1) / args.steps
        # per-step times on the GPU timeline: from one step's first event to
        # the next step's (the last step ends at eb1)
        nlin = len(linears)
        starts = [rec[i * nlin][2] for i in range(args.steps)] + [eb1]
        step_ms = np.array([starts[i].elapsed_time(starts[i + 1]) for i in range(args.steps)])
        pct = {f"p{q}": round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)}
        per = {}
        for name, fmt, e0, e1, e2 in rec:
            d = per.setdefault(name, {"fmt": fmt, "quant_ms": 0.0, "gemm_ms": 0.0})
            d["quant_ms"] += e0.elapsed_time(e1) / args.steps
            d["gemm_ms"] += e1.elapsed_time(e2) / args.steps
        results[sweep] = {"ms_per_step": ms, "wall_ms_per_step": 1e3 * wall / args.steps, "step_ms_pct": pct,
                          "instrumented_ms_per_step": ms_instr,
                          "tops": total_flops / (ms * 1e-3) / 1e12, "per_linear": per}
        print(f"[bench] {sweep}: {ms:.3f} ms/step, {results[sweep]['tops']:.1f} TOPS", file=sys.stderr,
              flush=True)

    head = results[chosen[0]]
    # dominant kernel of the headline step: the qgemm variant with the most time
    kern = {}
    for name, d in head["per_linear"].items():
        k = GEMM_OF[d["fmt"]]
        kk = kern.setdefault(k, {"ms": 0.0, "flops": 0.0, "launches": 0, "shapes": []})
        kk["ms"] += d["gemm_ms"]
        kk["flops"] += flops[name]
        kk["launches"] += 1
        kk["shapes"].append(next((K, N) for n, K, N in linears if n == name))
    dom = max(kern, key=lambda k: kern[k]["ms"])
    dk = kern[dom]
    achieved = dk["flops"] / (dk["ms"] * 1e-3) / 1e12
    # HBM bytes per call of the dominant GEMM from the committed counter runs
    # (FETCH_SIZE + WRITE_SIZE, copy-calibrated), while its sources match.  A
    # call is one data-parallel kernel plus, when the last wave is split along
    # K, the slice kernel and the reduce kernel: the dispatches of exactly
    # those grids are summed per call and averaged over the step's calls.
    from video_diffusion_transformer_block_amd import profiling
    rec = profiling.load_traffic(os.path.join(ROOT, "profiles", "traffic_5b_mixed.json"))
    afmt = {"qgemm_w4a4": 0, "qgemm_w4a8": 1}.get(dom)
    traffic = (gemm_call_traffic(rec, afmt, M, dk["shapes"])
               if rec is not None and afmt is not None else None)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_FP16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP16_MFMA_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per call (HBM/fabric, FETCH_SIZE+WRITE_SIZE)",
                "avg_launch_us": round(1e3 * dk["ms"] / dk["launches"], 1),
                "launch": "one GEMM call: data-parallel kernel (+ K-slice and reduce kernels for a split last wave)",
                "flops_per_launch": dk["flops"] / dk["launches"],
                "note": "exact NVFP4/INT8 operands run on the fp16 MFMA (the peak used); "
                        f"same rate vs fp8 {PEAK_FP8_TFLOPS:.0f}, fp4 {PEAK_FP4_TFLOPS:.0f} TFLOP/s: "
                        f"{achieved / PEAK_FP8_TFLOPS:.3f}, {achieved / PEAK_FP4_TFLOPS:.3f}"}

    # the MX GEMMs against their own peaks (FP4 10.1 PF for MXFP4 x MXFP4, FP8
    # 5.0 PF for MXFP8 x MXFP4), per activation format over the MX sweeps run
    mx_roof = {}
    for sweep, v in results.items():
        for name, d in v["per_linear"].items():
            if d["fmt"] in MX_PEAK:
                m = mx_roof.setdefault(d["fmt"], {"ms": 0.0, "flops": 0.0, "launches": 0})
                m["ms"] += d["gemm_ms"]
                m["flops"] += flops[name]
                m["launches"] += 1
    for fmt, m in mx_roof.items():
        ach = m["flops"] / (m["ms"] * 1e-3) / 1e12
        mx_roof[fmt] = {"bound": "mfma", "kernel": f"qgemm_mx_kernel<{'true' if fmt == 'mxfp8' else 'false'}, *>",
                        "achieved": round(ach, 1), "peak": MX_PEAK[fmt], "unit": "TFLOP/s",
                        "frac": round(ach / MX_PEAK[fmt], 4), "avg_launch_us": round(1e3 * m["ms"] / m["launches"], 1),
                        "launches": m["launches"]}

    # quantize pass alone (tensor amax supplied: the single fused kernel), HBM bound
    qroof = measure_quantize(torch, V, X, M, args.steps, want_mx)
    if rec is not None:
        for q in qroof.values():
            e = rec["kernels"].get(q["kernel"], {}).get("grids", {}).get(str(q["grid_work_items"]))
            if e is not None:
                q["traffic"] = round(e["bytes"])

    if args.calibration_copy:
        src = torch.ones(256 << 20, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    bsroof = measure_block_stats(torch, V, Xblk, Y["ffn_down"], M * hidden, args.steps)
    bf16ctx = measure_bf16_context(torch, X, host, linears, M, args.steps, up)
    stress = None if args.no_stress else measure_1080p(torch, V, args.steps)
    ffn_fusion = measure_ffn_fusion(torch, V, X, WM, M, args.steps) if want_mx else None

    dyn = None if args.no_dyn else measure_dyn(torch, V, synth)
    dmpq = measure_dmpq(V)
    cpu = None if args.no_cpu_baseline else cpu_baseline(host, M, args.cpu_rows)

    line = {
        "metric": "fused Hadamard-quant + W4A4/W4A8 GEMM TOPS at 5B shapes; % MFMA peak",
        "value": round(head["tops"], 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA on exactly decoded NVFP4/INT8 operands, f32 accumulate",
        "data": "synthetic: seeded Laplace(0,1) activations with 0.5% channels x30, N(0,0.02) weights",
        "config": {"workload": "CogVideoX-5B-shaped DiT block linears, M=17776 tokens, hidden 3072, "
                               "W4A6 mix (QKV+FFN-down NVFP4, out+FFN-up INT8), Hadamard block 64",
                   "M": M, "hidden": hidden, "had_block": HAD_BLOCK,
                   "linears": {n: [K, N] for n, K, N in linears}, "assignment": MIXED},
        "pct_fp16_mfma_peak": round(100 * head["tops"] / PEAK_FP16_MFMA_TFLOPS, 2),
        "roofline": roofline,
        "quantize_roofline": qroof,
        "mx_gemm_roofline": mx_roof or None,
        "block_stats_roofline": bsroof,
        "bf16_context": bf16ctx,
        "stress_1080p": stress,
        "ffn_fusion": ffn_fusion,
        "step_ms_pct": head["step_ms_pct"],
        "step_ms_pct_note": "per-step spread and per-call times come from a second pass of the same steps with "
                            "HIP events around every call (instrumented_ms_per_step); ms_per_step and value "
                            "come from the steps timed without them",
        "sweeps": {k: {"tops": round(v["tops"], 2), "ms_per_step": round(v["ms_per_step"], 4),
                       "instrumented_ms_per_step": round(v["instrumented_ms_per_step"], 4),
                       "step_ms_pct": v["step_ms_pct"],
                       "gemm_tflops": round(total_flops / (sum(d["gemm_ms"] for d in v["per_linear"].values())
                                                           * 1e-3) / 1e12, 1),
                       "per_linear_ms": {n: [round(d["quant_ms"], 4), round(d["gemm_ms"], 4)]
                                         for n, d in v["per_linear"].items()},
                       # the per-layer pipeline figure: 2MNK / (quantize + GEMM)
                       "per_linear_tops": {n: round(flops[n] / ((d["quant_ms"] + d["gemm_ms"]) * 1e-3) / 1e12, 1)
                                           for n, d in v["per_linear"].items()}}
                   for k, v in results.items()},
        "dyn_schedule": dyn,
        "dmpq_step": dmpq,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def bench_lib():
    """libvdtq_bench.so: plain streaming passes that move a launch's bytes
    with no arithmetic (the measured ceilings); not part of the library."""
    import ctypes
    path = os.path.join(ROOT, "video_diffusion_transformer_block_amd", "libvdtq_bench.so")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.vdtq_bench_stream_rows.restype = i32
    L.vdtq_bench_stream_rows.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    L.vdtq_bench_stream_3r1w.restype = i32
    L.vdtq_bench_stream_3r1w.argtypes = [vp, vp, vp, vp, i64, vp]
    return L


# bytes a quantize launch writes per 64-element chunk (codes, scales) and per row
STREAM_SHAPE = {"nvfp4": (32, 4, 0), "int8": (64, 0, 4), "mxfp4": (32, 2, 0), "mxfp8": (64, 2, 0)}


def measure_dmpq(V, blocks=30, steps=50, reps=20):
    """The host scheduler alone: dmpq_step over 30 blocks x 50 steps of
    seeded statistics (Gamma around the threshold, delta similarity around
    tau, an occasional outlier spike), repeated; microseconds per call
    through the ctypes binding, next to the cost of a trivial call through
    the same binding (vdtq_outlier_ratio), which bounds the marshalling."""
    rng = np.random.default_rng(9)
    n = blocks * steps
    g = 0.1 * np.exp(rng.normal(0.0, 0.5, n))
    r = 0.05 * np.exp(rng.normal(0.0, 0.7, n))
    stats = []
    for i in range(n):
        sin2 = 1.0e4
        sd2 = (g[i] ** 2) * sin2
        sp2 = 1.0e2
        sdd2 = (r[i] ** 2) * sp2
        stats.append([sd2, sin2, sdd2, sp2, 30.0, 1.0e4, 31.0, 1.0e4])
    ratio = np.where(rng.random(n) < 0.01, 1.0e4, 10.0)
    params = V.dmpq_params(gamma=0.1, tau=0.05, tau_acc=0.15, rho=1000.0)
    acts = [0, 0, 0, 0]
    t0 = time.perf_counter()
    for _ in range(reps):
        states = [V.dmpq_state() for _ in range(blocks)]
        last = [None] * blocks
        for t in range(steps):
            for b in range(blocks):
                i = t * blocks + b
                a = V.dmpq_step(params, states[b], last[b], float(ratio[i]))
                acts[a] += 1
                last[b] = None if a == 0 else stats[i]
    dt = time.perf_counter() - t0
    calls = reps * n
    t1 = time.perf_counter()
    for i in range(calls):
        V.outlier_ratio(30.0, 1.0e4, 1000)
    dt_floor = time.perf_counter() - t1
    return {"us_per_call": round(1e6 * dt / calls, 3), "calls": calls,
            "trivial_binding_call_us": round(1e6 * dt_floor / calls, 3),
            "actions": {"skip": acts[0], "nvfp4": acts[1], "int8": acts[2], "bf16": acts[3]},
            "note": "host only, through the ctypes binding (8 statistics marshalled per call); "
                    "the C function itself is a few comparisons per call"}


def measure_dyn(torch, V, synth, blocks=30, steps=50, M=4446, hidden=1920):
    """The closed-loop schedule study (30 blocks x 50 denoising steps, 4446
    tokens, hidden 1920) driven by dmpq_step, with the real linear on every
    computed block-step: the block's QKV projection (1920 -> 5760) runs at the
    precision the scheduler chose (NVFP4 -> W4A4, INT8 -> W4A8, BF16 -> the
    W4A16 fallback); a skipped block reuses its cached delta.  Block 0's input
    is Laplace(0, 1) with 0.5% of the channels x30; each computed block adds
    a smooth seeded residual plus decaying noise; three (block, step) pairs
    carry one channel x300.  Inputs and weights come from torch's seeded GPU
    generator.  The same loop is run again with every block-step forced to
    the BF16 fallback and no skip, for the reference; once more with the
    delta cache in MXFP8 (block_stats_mx8; a skipped block adds the
    dequantized cached delta); and once in bit-budget mode (each step's
    Gamma threshold from dmpq_budget_gamma for an average of 6 activation
    bits over the ranked blocks); and once with depth-aware skip thresholds
    (tau and tau_acc scaled from 1/2 at the first block to 3/2 at the last,
    dmpq_depth_params).  Times are HIP events around each computed block's
    quantize + GEMM."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)

    def laplace(shape, seed):
        gen.manual_seed(seed)
        e1 = torch.empty(shape, device=dev).exponential_(generator=gen)
        e2 = torch.empty(shape, device=dev).exponential_(generator=gen)
        return e1 - e2

    sched = synth.dyn_schedule(blocks, steps, M, hidden)
    ch = torch.from_numpy(synth.outlier_channels(hidden, synth.n_outliers(hidden), 3000)).to(dev)
    U = [laplace((M, hidden), 4000 + b) for b in range(blocks)]
    noise = []
    for b in range(blocks):
        gen.manual_seed(5000 + b)
        noise.append(torch.randn(M * hidden, generator=gen, device=dev))
    Wq = []
    for b in range(blocks):
        gen.manual_seed(2000 + b)
        w = (torch.randn((3 * hidden, hidden), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        Wq.append(V.hadamard_quantize(w, HAD_BLOCK, "nvfp4"))
    Ybuf = torch.empty((M, 3 * hidden), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * M * hidden * 3 * hidden
    fmt_of = {V.ACT_NVFP4: "nvfp4", V.ACT_INT8: "int8", V.ACT_BF16: "bf16"}

    def deq_mx8(c):
        # the cached MXFP8 delta as fp32 [M, hidden] (the skipped block's residual)
        v = c.q.view(torch.float8_e4m3fn).float().view(-1, 32) * torch.exp2(c.scales.float() - 127.0)[:, None]
        return v.view(M, hidden)

    def step_gamma(states, last, avg_bits):
        # bit-budget mode: this step's threshold from the Gamma_{t-1} of the
        # blocks that have one (a block computed last step: its new Gamma;
        # otherwise the Gamma it holds)
        gs = []
        for b in range(blocks):
            if last[b] is not None:
                d2, i2 = float(last[b][0]), float(last[b][1])
                gs.append((0.0 if d2 == 0.0 else math.inf) if i2 == 0.0 else math.sqrt(d2 / i2))
            elif states[b].has_gamma:
                gs.append(states[b].gamma_prev)
        return V.dmpq_budget_gamma(gs, avg_bits)

    def run(params, cache_fmt="bf16", budget=None, profile=None):
        states = [V.dmpq_state() for _ in range(blocks)]
        last = [None] * blocks
        cache = [None] * blocks
        acts = []
        spare = [None if cache_fmt == "mxfp8" else torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
                 for _ in range(blocks)]
        counts = {"skip": 0, "nvfp4": 0, "int8": 0, "bf16": 0}
        events = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            p_t = params
            if budget is not None:
                p_t = V.dmpq_params(gamma=step_gamma(states, last, budget), tau=params.tau, tau_acc=params.tau_acc,
                                    rho=params.rho, tau_u=params.tau_u, warmup=params.warmup)
            x = laplace((M, hidden), 500 + t)
            x[:, ch] *= 30.0
            x = x.to(torch.bfloat16)
            for b in range(blocks):
                spike = sched["spikes"].get((b, t))
                if spike is not None:
                    x = x.clone()
                    x[:, spike] = (x[:, spike].float() * 300.0).to(torch.bfloat16)
                _, rs = V.block_stats(x, x, write_delta=False)
                rs = rs.cpu().numpy()
                p_tb = p_t if profile is None else V.dmpq_depth_params(p_t, b, blocks, *profile)
                act = V.dmpq_step(p_tb, states[b], last[b], V.outlier_ratio(rs[4], rs[5], M * hidden))
                acts.append(act)
                if act == V.ACT_SKIP:
                    counts["skip"] += 1
                    res = deq_mx8(cache[b]) if cache_fmt == "mxfp8" else cache[b].float()
                    out = (x.float() + res).to(torch.bfloat16)
                    last[b] = None
                else:
                    fmt = fmt_of[act]
                    counts[fmt] += 1
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    a = V.hadamard_quantize(x, HAD_BLOCK, fmt)
                    {"nvfp4": V.qgemm_w4a4, "int8": V.qgemm_w4a8, "bf16": V.qgemm_w4a16}[fmt](
                        a, Wq[b], None, "bf16", y=Ybuf)
                    e1.record()
                    events.append((fmt, e0, e1))
                    a_b, beta_b, phi_b = sched["params"][b]
                    smooth = float(np.float32(a_b * (1.0 + 0.5 * np.sin(np.pi * t / steps + phi_b))))
                    decay = float(np.float32(beta_b * np.exp(-t / 10.0)))
                    z = torch.roll(noise[b], (7919 * t) % (M * hidden)).view(M, hidden)
                    out = (x.float() + (U[b] * smooth + z * decay)).to(torch.bfloat16)
                    if cache_fmt == "mxfp8":
                        dnew, st = V.block_stats_mx8(x, out, cache[b], spare[b])
                    else:
                        dnew = spare[b]
                        _, st = V.block_stats(x, out, cache[b], dnew)
                    last[b] = st.cpu().numpy()
                    spare[b] = cache[b] if cache[b] is not None or cache_fmt == "mxfp8" else torch.empty_like(dnew)
                    cache[b] = dnew
                x = out
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {}
        for fmt, e0, e1 in events:
            per.setdefault(fmt, []).append(e0.elapsed_time(e1))
        total = sum(sum(v) for v in per.values())
        return counts, per, total, wall, acts

    p_dyn = V.dmpq_params(gamma=0.1, tau=0.05, tau_acc=0.15, rho=1000.0)
    p_ref = V.dmpq_params(gamma=0.1, tau=0.0, tau_acc=0.0, rho=-1.0)    # always computes, always BF16
    counts, per, total, wall, acts = run(p_dyn)
    rcounts, rper, rtotal, rwall, _ = run(p_ref)
    c8, per8, total8, wall8, acts8 = run(p_dyn, "mxfp8")
    same = float(np.mean(np.array(acts) == np.array(acts8)))
    cb, perb, totalb, wallb, _ = run(p_dyn, budget=6.0)
    depth_prof = (0.5, 1.5)
    cd, perd, totald, walld, actsd = run(p_dyn, profile=depth_prof)

    def skips_by_third(a):
        sk = (np.array(a).reshape(steps, blocks) == V.ACT_SKIP).sum(0)
        th = blocks // 3
        return [int(sk[:th].sum()), int(sk[th:2 * th].sum()), int(sk[2 * th:].sum())]

    def avg_bits(c):
        n = c["nvfp4"] + c["int8"] + c["bf16"]
        return round((4 * c["nvfp4"] + 8 * c["int8"] + 16 * c["bf16"]) / n, 3) if n else None
    print(f"[bench] dyn schedule: actions {counts}, linear path {total:.1f} ms vs {rtotal:.1f} ms all-BF16; "
          f"MXFP8 cache: actions {c8}, {100 * same:.1f}% of decisions unchanged; budget 6 bits: actions {cb}; "
          f"depth profile {depth_prof}: actions {cd}",
          file=sys.stderr, flush=True)
    return {"workload": f"closed loop, {blocks} blocks x {steps} steps, M={M}, hidden {hidden}, "
                        f"QKV {hidden}->{3 * hidden} at the scheduled precision",
            "params": {"gamma": 0.1, "tau": 0.05, "tau_acc": 0.15, "rho": 1000.0, "warmup": 2},
            "actions": counts,
            "linear_ms_per_call": {k: round(float(np.mean(v)), 4) for k, v in per.items()},
            "linear_tflops": {k: round(flops / (float(np.mean(v)) * 1e-3) / 1e12, 1) for k, v in per.items()},
            "linear_ms_total": round(total, 2),
            "all_bf16_linear_ms_total": round(rtotal, 2),
            "linear_speedup_vs_all_bf16": round(rtotal / total, 3) if total else None,
            "wall_s": round(wall, 2), "all_bf16_wall_s": round(rwall, 2),
            "avg_activation_bits": avg_bits(counts),
            "budget_w4a6": {"actions": cb, "avg_activation_bits": avg_bits(cb),
                            "avg_quantized_bits": round((4 * cb["nvfp4"] + 8 * cb["int8"]) / max(1, cb["nvfp4"] + cb["int8"]), 3),
                            "linear_ms_total": round(totalb, 2),
                            "linear_speedup_vs_all_bf16": round(rtotal / totalb, 3) if totalb else None},
            "skips_by_depth_third": skips_by_third(acts),
            "depth_profile": {"tau_scale_shallow_to_deep": list(depth_prof), "actions": cd,
                              "skips_by_depth_third": skips_by_third(actsd),
                              "avg_activation_bits": avg_bits(cd), "linear_ms_total": round(totald, 2),
                              "linear_speedup_vs_all_bf16": round(rtotal / totald, 3) if totald else None},
            "mxfp8_cache": {"actions": c8, "linear_ms_total": round(total8, 2),
                            "same_action_fraction": round(same, 4),
                            "cache_bytes_per_block": M * hidden * (1 + 1 / 32),
                            "bf16_cache_bytes_per_block": M * hidden * 2}}


def gemm_call_grids(M, N, K, cus=256):
    """Work-items of the kernels of one pipelined GEMM call, as the library's
    launcher plans it (256 x 256 tiles, 256-thread workgroups, at most one
    workgroup per CU): the data-parallel kernel, and for a split last wave
    the K-slice kernel and the reduce kernel (64 workgroups per tile)."""
    tiles = -(-M // 256) * -(-N // 256)
    nk = K // 128
    g = max(1, min(cus, 256))
    left = tiles % g
    slices = min(g // left, nk) if left else 0
    slice_nk = -(-nk // slices) if slices else 0
    if slices:
        slices = -(-nk // slice_nk)
    split = slices >= 2 and slice_nk + 3 < nk
    sk = left if split else 0
    return {"dp": (tiles - sk) * 256, "sk": sk * slices * 256 if split else 0, "reduce": sk * 64 * 256}


def gemm_call_traffic(rec, afmt, M, shapes):
    """Mean FETCH+WRITE bytes per GEMM call of activation format afmt (0
    NVFP4, 1 INT8) over the calls of the given (K, N) shapes at M tokens:
    per call, the record's per-dispatch bytes of its data-parallel, K-slice
    and reduce grids (None when a grid is missing from the record)."""
    k = rec["kernels"]

    def grid_bytes(prefix, grid):
        for name, e in k.items():
            if name.startswith(prefix) and str(grid) in e["grids"]:
                return e["grids"][str(grid)]["bytes"]
        return None

    per_call = []
    for K, N in shapes:
        g = gemm_call_grids(M, N, K)
        parts = [grid_bytes(f"qgemm_pipe_kernel<{afmt}, false", g["dp"])]
        if g["sk"]:
            parts += [grid_bytes(f"qgemm_pipe_kernel<{afmt}, true", g["sk"]),
                      grid_bytes(f"qgemm_reduce_kernel<{afmt}>", g["reduce"])]
        if any(b is None for b in parts):
            return None
        per_call.append(sum(parts))
    return round(sum(per_call) / len(per_call)) if per_call else None


def measure_1080p(torch, V, steps, M=13 * 68 * 120 + 226, hidden=3072, ffn=12288):
    """The 1080p stress workload: 49 frames at 1088x1920 -> 106080 latent
    tokens + 226 text tokens, hidden 3072, FFN 3072 -> 12288 -> 3072.  Each
    FFN linear runs both ways: NVFP4 quantize (tensor amax computed) + W4A4,
    and INT8 quantize + W4A8; each quantize pass is also timed alone with the
    amax supplied.  Activations are Laplace(0, 1) with 0.5% of the channels
    x30, weights N(0, 0.02), drawn by torch's seeded GPU generator (the
    parity tests take the numpy recipe on sampled rows).  HIP events around
    3 launches, median."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)

    def laplace(shape, seed):
        gen.manual_seed(seed)
        x = torch.empty(shape, device=dev).exponential_(generator=gen)
        x -= torch.empty(shape, device=dev).exponential_(generator=gen)
        return x

    def activations(K, seed):
        x = laplace((M, K), seed)
        gen.manual_seed(seed + 1)
        ch = torch.randperm(K, generator=gen, device=dev)[:round(0.005 * K)]
        x[:, ch] *= 30.0
        return x.to(torch.bfloat16)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(3, steps // 6)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        return float(np.median(times))

    res = {"workload": f"1080p FFN: M={M} tokens (13x68x120 + 226), {hidden} -> {ffn} -> {hidden}, "
                       "Laplace(0,1) activations with 0.5% channels x30, N(0,0.02) weights (torch generator)"}
    for name, K, N, seed in (("ffn_up", hidden, ffn, 7100), ("ffn_down", ffn, hidden, 7200)):
        x = activations(K, seed)
        gen.manual_seed(seed + 2)
        w = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        wq = V.hadamard_quantize(w, HAD_BLOCK, "nvfp4")
        del w
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        flops = 2.0 * M * N * K
        e = {}
        a4 = V.hadamard_quantize(x, HAD_BLOCK, "nvfp4")
        a8 = V.hadamard_quantize(x, HAD_BLOCK, "int8")
        q4 = timed(lambda: V.hadamard_quantize(x, HAD_BLOCK, "nvfp4", amax="given", out=a4))
        q4c = timed(lambda: V.hadamard_quantize(x, HAD_BLOCK, "nvfp4", out=a4))
        q8 = timed(lambda: V.hadamard_quantize(x, HAD_BLOCK, "int8", out=a8))
        g4 = timed(lambda: V.qgemm_w4a4(a4, wq, None, "bf16", y=y))
        g8 = timed(lambda: V.qgemm_w4a8(a8, wq, None, "bf16", y=y))
        elems = M * K
        e["quantize_nvfp4"] = {"us": round(1e3 * q4, 1), "gbs": round(QUANT_BYTES["nvfp4"] * elems / (q4 * 1e-3) / 1e9, 1),
                               "frac_hbm": round(QUANT_BYTES["nvfp4"] * elems / (q4 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        e["quantize_nvfp4_amax_computed_us"] = round(1e3 * q4c, 1)
        b8 = (QUANT_BYTES["int8"] + 4.0 / K) * elems
        e["quantize_int8"] = {"us": round(1e3 * q8, 1), "gbs": round(b8 / (q8 * 1e-3) / 1e9, 1),
                              "frac_hbm": round(b8 / (q8 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        e["w4a4"] = {"ms": round(g4, 4), "tflops": round(flops / (g4 * 1e-3) / 1e12, 1),
                     "frac_fp16_peak": round(flops / (g4 * 1e-3) / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4)}
        e["w4a8"] = {"ms": round(g8, 4), "tflops": round(flops / (g8 * 1e-3) / 1e12, 1),
                     "frac_fp16_peak": round(flops / (g8 * 1e-3) / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4)}
        res[name] = e
        del x, wq, y, a4, a8
        torch.cuda.empty_cache()
        print(f"[bench] 1080p {name}: nvfp4 quant {e['quantize_nvfp4']['us']} us, int8 quant "
              f"{e['quantize_int8']['us']} us, W4A4 {e['w4a4']['tflops']} / W4A8 {e['w4a8']['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    return res


def measure_bf16_context(torch, X, host, linears, M, steps, up):
    """Context row, not a target: the four linears as plain bf16 GEMMs in
    torch (hipBLASLt), Y = X W^T with the unquantized bf16 weights, the
    weight operand made contiguous as [K, N] first.  HIP events around 10
    launches, median per linear."""
    per = {}
    total_ms, total_flops = 0.0, 0.0
    for name, K, N in linears:
        wt = up(host[name][1]).t().contiguous()          # [K, N]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=X[name].device)
        torch.mm(X[name], wt, out=y)
        torch.cuda.synchronize()
        times = []
        for _ in range(max(3, steps // 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                torch.mm(X[name], wt, out=y)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 10)
        ms = float(np.median(times))
        f = 2.0 * M * N * K
        per[name] = {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
        total_ms += ms
        total_flops += f
        del wt, y
    return {"what": "torch.mm bf16 (hipBLASLt), unquantized weights, same shapes; context only",
            "per_linear": per, "gemm_ms": round(total_ms, 4),
            "tops": round(total_flops / (total_ms * 1e-3) / 1e12, 1)}


def measure_block_stats(torch, V, inp, out, n, steps):
    """block_stats over the 5B block's input and output (17776 x 3072) with
    the delta cache in bf16 (8 bytes per element: in, out, Delta_prev read,
    Delta_new written) and in MXFP8 (6 + 1/16 bytes per element), each
    reading the delta the previous launch wrote; HIP events around 20
    launches."""
    res = {}
    for cache, bpe in (("bf16", 8.0), ("mxfp8", 6.0 + 2 / 32)):
        if cache == "bf16":
            d0, _ = V.block_stats(inp, out)
            d1 = torch.empty_like(d0)
            run = lambda a, b: V.block_stats(inp, out, a, b)
        else:
            d0, _ = V.block_stats_mx8(inp, out)
            d1, _ = V.block_stats_mx8(inp, out)
            run = lambda a, b: V.block_stats_mx8(inp, out, a, b)
        run(d0, d1)
        torch.cuda.synchronize()
        times = []
        for _ in range(max(3, steps // 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(20):
                run(d0, d1) if i % 2 == 0 else run(d1, d0)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 20)
        us = 1e3 * float(np.median(times))
        gbs = bpe * n / (us * 1e-6) / 1e9
        if cache == "bf16":
            # the same bytes through a plain streaming pass (3 reads, 1 write)
            import ctypes
            BL = bench_lib()
            dsink = torch.empty_like(d0)
            st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            ptr = lambda t: ctypes.c_void_p(t.data_ptr())
            srun = lambda a, b: BL.vdtq_bench_stream_3r1w(ptr(inp), ptr(out), ptr(a), ptr(b), n, st())
            srun(d0, dsink)
            torch.cuda.synchronize()
            stimes = []
            for _ in range(max(3, steps // 4)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(20):
                    srun(d0, dsink) if i % 2 == 0 else srun(dsink, d0)
                e1.record()
                torch.cuda.synchronize()
                stimes.append(e0.elapsed_time(e1) / 20)
            cus = 1e3 * float(np.median(stimes))
            del dsink
        res[cache] = {"bound": "hbm", "kernel": ("block_stats_kernel<true> + block_stats_final_kernel" if cache == "bf16"
                                                else "block_stats_mx8_kernel + block_stats_final_kernel"),
                      "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                      "avg_launch_us": round(us, 2), "bytes_per_launch": bpe * n,
                      "cache_bytes": n * (2 if cache == "bf16" else 1 + 1 / 32)}
        if cache == "bf16":
            res[cache]["ceiling"] = {"what": "plain streaming pass, 3 bf16 reads + 1 write of n, no arithmetic",
                                     "avg_launch_us": round(cus, 2),
                                     "achieved": round(bpe * n / (cus * 1e-6) / 1e9, 1),
                                     "frac": round(bpe * n / (cus * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            res[cache]["frac_of_ceiling"] = round(cus / us, 4)
    return res


def hq_grid_work_items(M, K, fmt):
    """Work-items of one quantize launch, as the library's launcher sizes it:
    one 64-element chunk per thread for NVFP4 and MX; for INT8, whole rows
    per group of int8_threads(chunks per row) threads.  Keys the counter
    record."""
    cpr = (K + 63) // 64
    if fmt != "int8":
        return -(-M * cpr // 128) * 128
    threads = int8_threads(cpr)
    rpw = max(1, threads // cpr)
    return -(-M // rpw) * threads


def int8_threads(cpr):
    """Workgroup size of the INT8 quantize kernel for rows of cpr chunks of
    64 (the library's rule: 192 threads when their whole rows leave fewer
    lanes idle than 256 threads' do, else 256)."""
    r192, r256 = 192 // cpr, 256 // cpr
    return 192 if r192 >= 1 and r192 * cpr * 256 > r256 * cpr * 192 else 256


QUANT_BYTES = {"nvfp4": 2 + 0.5 + 1 / 16, "int8": 3.0, "mxfp4": 2 + 0.5 + 1 / 32, "mxfp8": 2 + 1 + 1 / 32}
QUANT_KERNEL = {"nvfp4": "hq_nvfp4_kernel<64, false>", "int8": "hq_int8_kernel<64, 192>",
                "nvfp4_amax": "hq_amax_kernel<64> + hq_amax_final_kernel + hq_nvfp4_kernel<64, false>",
                "mxfp4": "hq_mx_kernel<64, false>", "mxfp8": "hq_mx_kernel<64, true>"}


def measure_quantize(torch, V, X, M, steps, with_mx=False):
    """hadamard_quantize with the tensor amax supplied (the single fused
    kernel), and NVFP4 with the tensor amax computed (pre-pass, its final
    reduction and the pass: 2 more bytes per element, key nvfp4_amax).  The
    launches are captured in a graph and replayed, so the per-launch time
    (HIP events around the replays / launches) excludes host launch gaps.
    Each shape rotates over distinct copies of its inputs totalling at least
    1 GB (ten 109 MB copies of the three K = 3072 activations, three of the
    437 MB FFN-down input), four times the 256 MB last-level cache, so every
    launch reads its input from HBM.  Beside each pass, `ceiling` times a
    plain streaming kernel that moves exactly the same bytes per launch with
    no arithmetic (same grid shape of one 64-element chunk per thread, same
    rotation, same graph replay): the rate this launch size allows."""
    import ctypes
    BL = bench_lib()
    out = {}
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for K, names in ((3072, ["qkv", "out", "ffn_up"]), (12288, ["ffn_down"])):
        elems = M * K
        n_copies = max(3, -(-int(1.0e9) // (2 * elems)))
        srcs = [X[names[i % len(names)]].clone() for i in range(n_copies)]
        n_launch = 2 * n_copies
        for key in ("nvfp4", "nvfp4_amax", "int8") + (("mxfp4", "mxfp8") if with_mx else ()):
            fmt = "nvfp4" if key == "nvfp4_amax" else key
            bpe = QUANT_BYTES[fmt] + (2.0 if key == "nvfp4_amax" else 0.0)
            extra = 0 if fmt == "nvfp4" else 4 * M / elems
            # buffers allocated (and the tensor amax written) before capture
            outs = [V.hadamard_quantize(x, HAD_BLOCK, fmt) for x in srcs]
            amax = "given" if key == "nvfp4" else None

            def replay_us(launch):
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n_launch):
                        launch(i % n_copies)
                g.replay()
                torch.cuda.synchronize()
                times = []
                for _ in range(max(3, steps // 4)):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1) / n_launch)
                del g
                return 1e3 * float(np.median(times))

            us = replay_us(lambda j: V.hadamard_quantize(srcs[j], HAD_BLOCK, fmt, amax=amax, out=outs[j]))
            gbs = (bpe + extra) * elems / (us * 1e-6) / 1e9
            e = {"bound": "hbm", "kernel": QUANT_KERNEL[key], "achieved": round(gbs, 1),
                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                 "traffic": None, "avg_launch_us": round(us, 2),
                 "bytes_per_launch": (bpe + extra) * elems, "shape": [M, K],
                 "grid_work_items": hq_grid_work_items(M, K, fmt),
                 "rotation": f"{n_copies} distinct inputs, {n_copies * 2 * elems / 1e9:.2f} GB"}
            if key == "nvfp4_amax":
                e["note"] = ("algorithmic bytes (2 reads of X): the pass re-reads the tensor the pre-pass just "
                             "read, and up to 256 MB of that comes from the last-level cache, not HBM")
            else:
                cb, sb, rb = STREAM_SHAPE[fmt]
                chunks = elems // 64
                q = torch.empty(chunks * cb, dtype=torch.uint8, device=srcs[0].device)
                sc = torch.empty(max(1, chunks * sb), dtype=torch.uint8, device=srcs[0].device)
                rw = torch.empty(M, dtype=torch.int32, device=srcs[0].device)

                def stream_launch(j):
                    rc = BL.vdtq_bench_stream_rows(ctypes.c_void_p(srcs[j].data_ptr()), M, K, cb, sb, rb,
                                                   ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
                                                   ctypes.c_void_p(rw.data_ptr()), stream())
                    assert rc == 0, rc
                cus = replay_us(stream_launch)
                cgbs = (bpe + extra) * elems / (cus * 1e-6) / 1e9
                e["ceiling"] = {"what": "plain streaming pass, same bytes and launch size, no arithmetic",
                                "avg_launch_us": round(cus, 2), "achieved": round(cgbs, 1),
                                "frac": round(cgbs / PEAK_HBM_GBS, 4)}
                e["frac_of_ceiling"] = round(cus / us, 4)
                del q, sc, rw
            out[f"{key}_K{K}"] = e
            del outs
        del srcs
        torch.cuda.empty_cache()
    return out


def measure_ffn_fusion(torch, V, X, WM, M, steps):
    """FFN-up feeding FFN-down at the 5B shape (17776 x 3072 -> 12288, MXFP4
    weights, bias): the unfused chain qgemm_mx (bf16 Y) -> hadamard_quantize
    (GELU, Hadamard 64, MXFP4) against qgemm_mx_quant, which never writes Y;
    for MXFP8 activations (the W4A6 mix's FFN-up format) and MXFP4.  Each
    part is timed alone too (HIP events around 10 launches, median).  Also
    FFN-down's NVFP4 quantize of the same Y (tensor amax computed) with and
    without GELU."""
    N = WM["ffn_up"].q.shape[0]
    gen = torch.Generator(device=X["ffn_up"].device).manual_seed(77)
    bias = torch.randn(N, generator=gen, device=X["ffn_up"].device) * 0.1
    y = torch.empty((M, N), dtype=torch.bfloat16, device=X["ffn_up"].device)
    w = WM["ffn_up"]

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(3, steps // 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        return round(1e3 * float(np.median(times)), 1)

    res = {"workload": f"FFN-up {M}x3072 -> {N} + bias, GELU, Hadamard 64, MXFP4 FFN-down activation",
           "bf16_round_trip_bytes": 4 * M * N}
    q = V.hadamard_quantize(y, HAD_BLOCK, "mxfp4")
    res["quant_us"] = timed(lambda: V.hadamard_quantize(y, HAD_BLOCK, "mxfp4", out=q))
    res["quant_gelu_us"] = timed(lambda: V.hadamard_quantize(y, HAD_BLOCK, "mxfp4", gelu=True, out=q))
    # the headline format's FFN-down input in a model: NVFP4 with the tensor
    # amax computed, both passes applying GELU
    qn = V.hadamard_quantize(y, HAD_BLOCK, "nvfp4")
    res["nvfp4_quant_us"] = timed(lambda: V.hadamard_quantize(y, HAD_BLOCK, "nvfp4", out=qn))
    res["nvfp4_quant_gelu_us"] = timed(lambda: V.hadamard_quantize(y, HAD_BLOCK, "nvfp4", gelu=True, out=qn))
    for afmt in ("mxfp8", "mxfp4"):
        a = V.hadamard_quantize(X["ffn_up"], HAD_BLOCK, afmt)
        qf = V.qgemm_mx_quant(a, w, bias, "mxfp4", gelu=True)
        gemm = timed(lambda: V.qgemm_mx(a, w, bias, "bf16", y=y))
        chain = timed(lambda: (V.qgemm_mx(a, w, bias, "bf16", y=y),
                               V.hadamard_quantize(y, HAD_BLOCK, "mxfp4", gelu=True, out=q)))
        fused = timed(lambda: V.qgemm_mx_quant(a, w, bias, "mxfp4", gelu=True, out=qf))
        res[afmt] = {"gemm_bf16_us": gemm, "unfused_us": chain, "fused_us": fused,
                     "speedup": round(chain / fused, 3)}
        print(f"[bench] ffn fusion {afmt}: gemm {gemm} us, chain {chain} us, fused {fused} us", file=sys.stderr,
              flush=True)
    return res


def cpu_baseline(host, M, rows):
    """The oracle, as it stands, on a bounded sample of the same step: the
    first `rows` tokens of each of the four linears (NVFP4 amax over the
    sample), quantize + GEMM; weights prepared beforehand (offline, untimed)."""
    import oracle.quant as Q
    import oracle.gemm as G
    cores = len(os.sched_getaffinity(0))
    prepped = {n: Q.prepare_weight(w, HAD_BLOCK) for n, (x, w) in host.items()}
    t0 = time.perf_counter()
    flops = elems = 0.0
    tq = tg = 0.0
    for name, (x, w) in host.items():
        xs = x[:rows]
        wq, ws, wgs = prepped[name]
        fmt = MIXED[name]
        t1 = time.perf_counter()
        a = Q.hadamard_quantize(xs, HAD_BLOCK, fmt)
        t2 = time.perf_counter()
        if fmt == "nvfp4":
            G.qgemm_w4a4(a["q"], a["scales"], a["gs"], wq, ws, wgs, None, "bf16")
        else:
            G.qgemm_w4a8(a["q"], a["scales"], wq, ws, wgs, None, "bf16")
        tq += t2 - t1
        tg += time.perf_counter() - t2
        flops += 2.0 * rows * w.shape[0] * w.shape[1]
        elems += xs.size
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "quantize_elements_per_s": round(elems / tq, 1), "gemm_fp64_flop_per_s": round(flops / tg, 1),
            "sample": f"first {rows} of {M} tokens of each of the 4 linears (mixed W4A6 assignment), "
                      "quantize + GEMM; numpy float64 GEMM, weights decoded per call"}


if __name__ == "__main__":
    main()
