#!/usr/bin/env python3
"""Throughput of the LLM.int8() linear layer on one MI355X.

One step = one int8_linear_forward call (outlier detection, masked row
quantization + gathers, fused int8/fp16 product with epilogue) on the 13B-scale
first feed-forward layer: X fp16 [2048, 5120] with 6 planted outlier columns,
W [20480, 5120] held as CB/SCB (quantized once, outside the timed region).
Inputs are seeded synthetic data resident in HBM before timing starts.

Prints one JSON line: effective TOPS (2*T*N*K per second over the whole
call, from K back-to-back calls with no instrumentation, rotating over
copies of the inputs so that the last-level cache holds none of a step's
operands; the same K calls on one copy give the warm figure beside it), the
roofline entry of the dominant kernel (the fused product, timed over another
run of the K calls by HIP events the library records around it on the same
stream), the fp16 torch linear on the same shape and copies for comparison,
and the CPU oracle timed on this host's cores.
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

PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, 2.5 PFLOP/s
CSRC = "int8_mixed_precision_detect_amd/csrc/"
# the sources of the product kernel that runs for T tokens (T <= 4: the
# row-streaming one; else the tiled one)
GEMM_SOURCES = {"gemv": [CSRC + "k_gemv.hip", CSRC + "common.h", CSRC + "kernels.h"],
                "tiled": [CSRC + "k_gemm_i8.hip", CSRC + "common.h", CSRC + "kernels.h"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_{}_traffic.txt")  # per workload


def product_path(T: int) -> str:
    return "gemv" if T <= 4 else "tiled"


def kernel_fingerprint(path: str = "tiled") -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES[path]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


ENTRY = {"int8": "int8_linear_forward", "fp16w": "int8_linear_forward_fp16w",
         "zeropoint": "int8_linear_forward_zeropoint"}

WORKLOAD_DESC = {
    "tiny": "tiny (16 tokens, 64 x 64 LLM.int8() linear)",
    "6.7b": "6.7b-scale first FF layer (LLM.int8() linear)",
    "13b": "13b-scale first FF layer (LLM.int8() linear)",
    "13b-down": "13b-scale second FF layer, down projection K = 4h (LLM.int8() linear)",
    "13b-attn": "13b-scale attention projection K = N = h (LLM.int8() linear)",
    "175b": "175b-scale first FF layer (LLM.int8() linear)",
    "175b-n8": "175b-scale first FF layer, one GPU's 1/8 of the output channels (LLM.int8() linear)",
    "decode1": "decode1-scale first FF layer (LLM.int8() linear)",
    "decode8": "decode8-scale first FF layer (LLM.int8() linear)",
    "decode32": "decode32-scale first FF layer (LLM.int8() linear)",
}


def profile_tag(workload: str, layer: str) -> str:
    return workload if layer == "int8" else f"{workload}-{layer}"


def read_traffic(workload: str, layer: str = "int8", T: int = 2048):
    """HBM bytes per launch of the product kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel source
    (T picks the kernel whose sources are hashed)."""
    tag = profile_tag(workload, layer)
    path = TRAFFIC_FILE.format(tag)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    if kv.get("kernel_fingerprint") != kernel_fingerprint(product_path(T)) or kv.get("workload") != tag:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(d, cols: int, reps: int, layer: str = "int8"):
    """The oracle as it stands, on all rows and the first `cols` output channels."""
    import numpy as np
    import oracle.llm_int8 as O
    X, W, bias, thr = d["X"], d["W"], d["bias"], d["threshold"]
    T, K = X.shape
    CB, SCB = O.quantize_weight(W[:cols])          # load-time step, not timed
    b = None if bias is None else bias[:cols]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if layer == "fp16w":
            O.linear_forward_fp16w(X, W[:cols], b, thr)
        elif layer == "zeropoint":
            O.linear_forward_zeropoint(X, CB, SCB, b, thr)
        else:
            O.linear_forward(X, CB, SCB, b, thr)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    return {"value": 2.0 * T * cols * K / t / 1e12, "unit": "TOPS",
            "cores": threads or cores, "host_cores": cores, "kind": "oracle",
            "sample": f"full forward of the CPU oracle (NumPy, float64 BLAS) on all {T} rows and "
                      f"the first {cols} of {W.shape[0]} output channels, median of {reps} runs "
                      f"({t:.2f} s each, {sum(times):.1f} s in all)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clocks take some 20-40 ms of sustained work to settle: the
    # default warmup (~25 ms at the 13B shape) keeps that ramp out of the
    # timed calls
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="13b")
    ap.add_argument("--layer", choices=("int8", "fp16w", "zeropoint"), default="int8",
                    help="int8 weight (default); fp16 weight kept and quantized per call; "
                         "zero-point activation codes")
    ap.add_argument("--copies", type=int, default=3,
                    help="rotate this many copies of X/CB/SCB/Y so the 256 MB last-level "
                         "cache cannot hold one step's inputs from the step before")
    ap.add_argument("--cpu-cols", type=int, default=20480)
    ap.add_argument("--cpu-reps", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus must be 1 "
              f"(got {args.gpus})", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import int8_mixed_precision_detect_amd as i8
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    T, K, N = wl.T, wl.K, wl.N
    d = make_inputs(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    copies = max(1, args.copies)
    Xs, CBs, SCBs, Ys, Ws, RSs = [], [], [], [], [], []
    Wd = torch.from_numpy(d["W"]).to(dev)
    for _ in range(copies):
        Xs.append(torch.from_numpy(d["X"]).to(dev))
        CB, SCB = i8.quantize_weight(Wd)
        CBs.append(CB)
        SCBs.append(SCB)
        Ys.append(torch.empty((T, N), dtype=torch.float16, device=dev))
        if args.layer == "fp16w" or not args.no_fp16:
            Ws.append(Wd.clone())
        if args.layer == "zeropoint":
            RSs.append(i8.weight_rowsum(CB))
    bias = None if d["bias"] is None else torch.from_numpy(d["bias"]).to(dev)
    ws = i8.alloc_workspace(T, N, K, None, dev)
    torch.cuda.synchronize()

    def step(s):
        c = s % copies
        if args.layer == "fp16w":
            i8.linear_forward_fp16w(Xs[c], Ws[c], bias, wl.threshold, workspace=ws, out=Ys[c],
                                    CB=CBs[c], SCB=SCBs[c])
        elif args.layer == "zeropoint":
            i8.linear_forward_zeropoint(Xs[c], CBs[c], SCBs[c], RSs[c], bias, wl.threshold,
                                        workspace=ws, out=Ys[c])
        else:
            i8.linear_forward(Xs[c], CBs[c], SCBs[c], bias, wl.threshold, workspace=ws, out=Ys[c])

    # the fp16 comparator on the same shape (torch.nn.functional.linear, i.e.
    # hipBLASLt), rotated over the same number of input/weight copies, then on
    # one copy; it runs before the int8 steps
    fp16 = None
    if not args.no_fp16:
        F = torch.nn.functional
        reps = max(10, args.steps // 2)

        def fp16_ms(rotate):
            for r in range(3):
                F.linear(Xs[r % copies], Ws[r % copies], bias)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(reps):
                c = r % copies if rotate else 0
                F.linear(Xs[c], Ws[c], bias)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        fp16 = (fp16_ms(True), fp16_ms(False))

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    code, n_o = i8.linear_status(ws)
    if code != 0:
        raise RuntimeError(f"forward reported status {code}")

    # throughput: K steps with nothing else on the stream
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(s)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / args.steps

    # the same K steps on copy 0 only: inputs partly held in the 256 MB
    # last-level cache from the step before (the warm figure; `value` is the
    # rotated one above)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(0)
    stop.record()
    torch.cuda.synchronize()
    warm_ms_per_step = start.elapsed_time(stop) / args.steps

    # per-kernel durations: the same K steps again, with the library's HIP
    # events recorded on the launch stream around each stage (an event
    # between two kernels leaves the queue idle for a few microseconds, so
    # this pass is kept out of the throughput figure above)
    i8.profile_enable(True)
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    stage_ms, calls = i8.profile_read()
    i8.profile_enable(False)
    if calls != args.steps:
        raise RuntimeError(f"timed {calls} calls, expected {args.steps}")
    stage_avg = [m / max(calls, 1) for m in stage_ms]

    # per-call spread: the same calls once more, each bracketed by its own
    # events on the launch stream (torch's current stream)
    per_call = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for s, (e0, e1) in enumerate(evs):
        e0.record()
        step(s)
        e1.record()
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    pct = lambda q: round(per_call[min(len(per_call) - 1, int(q * (len(per_call) - 1) + 0.5))], 2)

    ops = 2.0 * T * N * K
    tops = ops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = stage_avg[2]
    traffic = read_traffic(args.workload, args.layer, T)
    n_pad = -(-n_o // 32) * 32
    ldq = -(-K // 64) * 64
    # the fp16 outlier product, the method's own work beside the int8 one
    f16_flops = 2.0 * T * N * n_o
    # step 2 builds the outlier weights Wo unless the few-token tiles take
    # them from their own CB stream (int8 layer, T <= 32, n_o <= 128)
    wo_in_prep = T > 32 or n_o > 128 or args.layer != "int8"
    # one to eight tokens, absmax layer: steps 1-2 run as one launch of one
    # workgroup (no mask, no Wo; the product takes every outlier set from CB
    # itself)
    row_prep = T <= 8 and args.layer == "int8" and K % 16 == 0 and K <= 16384
    if row_prep:
        wo_in_prep = False
    if T <= 32:
        # few tokens: the product streams CB once -- an HBM-bound kernel;
        # algorithmic bytes per launch: reads CB, Xq, Xo, SCB, sx, bias;
        # writes Y, and picks Wo out of the CB stream (writing it) when step
        # 2 did not build it, else reads it back
        gemm_bytes = (N * K + T * ldq + 2 * T * n_pad + 4 * N + 4 * T
                      + (2 * N if d["bias"] is not None else 0) + 2 * N * n_pad + 2 * T * N)
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": ("k_gemv, row-streaming (int8 product + epilogue)" if T <= 4 else
                               "k_gemm_i8, few-token tiles (int8 product + epilogue)"),
                    "avg_ms": round(gemm_ms, 5), "algorithmic_bytes_per_launch": gemm_bytes}
    else:
        # int8 ops against the int8 peak; the fp16 outlier flops against the
        # fp16 peak; frac is time-weighted: the time both would take at their
        # peaks over the measured time (the int8 ops alone when n_o is small)
        achieved = ops / (gemm_ms * 1e-3) / 1e12
        t_min = ops / (PEAK_INT8_TOPS * 1e12) + f16_flops / (PEAK_FP16_TFLOPS * 1e12)
        splits = i8.workspace_layout(T, N, K)["splits"]
        kname = ("k_gemm_i8 (fused int8 product + epilogue)" if splits == 1 else
                 f"k_gemm_i8, K split {splits} ways (int8 partial tiles, then combine + epilogue)")
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                    "unit": "TFLOP/s", "frac": round(t_min / (gemm_ms * 1e-3), 4),
                    "traffic": traffic, "kernel": kname,
                    "avg_ms": round(gemm_ms, 5), "algorithmic_ops_per_launch": ops,
                    "fp16_outlier_flops_per_launch": f16_flops,
                    "int8_only_frac": round(achieved / PEAK_INT8_TOPS, 4)}
    detect_bytes = 2.0 * T * K
    if args.layer == "fp16w":
        # (the per-call weight quantization runs in the detect stage: reads
        # W, writes CB and SCB)
        detect_bytes += 2.0 * N * K + N * K + 4 * N
    # step-2 prep: read X, write Xq (ldq = K rounded to 64), sx and Xo; the
    # outlier weights when it builds them (a gather of CB[:, O], of W[:, O]
    # in fp16 for the fp16-weight layer, and an fp16 write); the zero-point
    # layer's row offsets and per-channel outlier code sums
    quant_bytes = 2.0 * T * K + T * ldq + 4 * T + 2 * T * n_pad
    if wo_in_prep:
        quant_bytes += N * n_o * (2 if args.layer == "fp16w" else 1) + 2 * N * n_pad
    if args.layer == "zeropoint":
        quant_bytes += 4 * T + 4 * N

    result = {
        "metric": f"effective TOPS (2TNK/s) of {ENTRY[args.layer]} at T={T}; % int8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC.get(args.workload, args.workload),
                   "T": T, "K": K, "N": N, "threshold": wl.threshold, "n_outliers": n_o,
                   "bias": d["bias"] is not None, "buffer_copies": copies,
                   "k_splits": i8.workspace_layout(T, N, K)["splits"], "layer": args.layer},
        "roofline": roofline,
        "stages_ms": ({"steps_1_2_one_launch": round(stage_avg[0], 5),
                       "product": round(stage_avg[2], 5), "whole_call": round(stage_avg[3], 5)}
                      if row_prep else
                      {"detect": round(stage_avg[0], 5), "quantize_gather": round(stage_avg[1], 5),
                       "product": round(stage_avg[2], 5), "whole_call": round(stage_avg[3], 5)}),
        "stages_hbm_frac": ({"steps_1_2_one_launch": round(
                                quant_bytes / (stage_avg[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                            if row_prep else {
            "detect": round(detect_bytes / (stage_avg[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "quantize_gather": round(quant_bytes / (stage_avg[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}),
        "pct_int8_peak_whole_call": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "per_call_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "calls": len(per_call)},
        "cold_warm_ms_per_step": {"rotated_copies": round(ms_per_step, 5),
                                  "same_buffers": round(warm_ms_per_step, 5)},
    }
    if fp16 is not None:
        result["fp16_linear"] = {"ms": round(fp16[0], 5),
                                 "tflops": round(ops / (fp16[0] * 1e-3) / 1e12, 2),
                                 "int8_over_fp16_time": round(ms_per_step / fp16[0], 4),
                                 "same_buffers_ms": round(fp16[1], 5),
                                 "rotated_copies": copies}

    if args.copy_calib_mb > 0:
        nbytes = args.copy_calib_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nbytes

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, min(args.cpu_cols, N), max(1, args.cpu_reps),
                                              args.layer)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
