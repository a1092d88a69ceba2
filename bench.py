#!/usr/bin/env python3
"""Benchmark of the rotated INT8 linear layer on one MI355X.

One step = one int8_linear call over the whole input (rotate+quantize kernel,
then the INT8 MFMA GEMM with the fused dequantizing epilogue), inputs already
resident in HBM.  The weights are prepared offline (rotated, quantized and
stored in the K-sliced layout: int8_linear_sliced; --row-major-weights runs
int8_linear on the row-major codes instead, same results).  The reported value is 2*M*N*K / step time in TOP/s (INT8
ops; the rotation and quantization are inside the timed step).

Prints ONE JSON line.  Besides the headline it carries:
  roofline      the GEMM kernel (dominant) against the dense INT8 MFMA peak,
                its duration measured with HIP events on the launch stream;
  kernels       both kernels' average durations, TOP/s or GB/s and fractions;
  cpu_baseline  the plain C oracle timed on the host cores over a bounded
                sample of the same workload (the leading rows), and the GPU
                output of those rows compared with it.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 3]
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

PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, published (5.0 POP/s)
PEAK_FP6_TFLOPS = 10100.0      # MI355X dense FP6/FP4 MFMA, published (10.1 PFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published (8 TB/s)
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, published (2.5 PFLOP/s)
# int8_attention: half its operations on the INT8 matrix cores (Q K^T), half on
# the BF16 ones (P V): the combined dense peak is 1 / (0.5 / 5000 + 0.5 / 2500)
PEAK_ATTN_TOPS = 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_BF16_TFLOPS)
# attention workload: 40 heads of dimension 128 (a 14B-class video DiT block), one 16384-token sequence
ATTN_BH, ATTN_L, ATTN_D = 40, 16384, 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_i8_traffic.json")
GEMM_SRC = os.path.join(ROOT, "quantized_diffusion_amd", "csrc", "gemm_i8.hip")
# The pages' single-call figure for M32700/K5376/N16128 on an RTX 5090 D v2
# (SGLang PR "Tune Kitchen INT8 row splitting for SM120", Benchmark table):
# 10.5752 ms.  Context only, another machine.
PAGE_MS = {3: 10.5752, 2: 2.7743}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(path: str) -> str:
    """Hash of the kernel source's code (comments and blank lines dropped)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in code if ln).encode()).hexdigest()[:16]


def load_traffic(workload_name: str):
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != kernel_hash(GEMM_SRC):
        return None                      # counters were taken on another version of the kernel
    return d.get("workloads", {}).get(workload_name, {}).get("hbm_bytes_per_launch")


def time_launches(fn, n, torch):
    """Average duration (ms) of fn() over n back-to-back launches, timed with one pair of HIP
    events on the current stream (the stream the binding launches on)."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def cpu_baseline(x_dev, y_dev, wq_dev, sw_dev, b_bits, w, torch, budget_s: float, act: int = 0,
                 codes: bool = False):
    """Time the oracle on the leading rows of the same workload; check those rows."""
    import numpy as np

    import oracle
    O = oracle.default()
    int4 = w.kind == "w4a4"
    wq = wq_dev.cpu().numpy()
    if int4 and not codes:
        wq = O.unpack_int4(wq, w.K)     # packed weights -> INT4 codes in INT8 storage
    sw = sw_dev.cpu().numpy()

    def run(rows):
        x = x_dev[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        y = O.linear(x, wq, sw, b_bits, qmax=7 if int4 else 127, act=act)
        return time.perf_counter() - t0, y

    t_small, _ = run(16)
    rows = int(min(w.M, max(16, 16 * budget_s / max(t_small, 1e-3))))
    rows = min(rows, 20000)       # about 10-15 s of oracle work on the host's cores
    t, y_or = run(rows)
    y_gpu = y_dev[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    same = y_gpu == y_or
    within = True
    for r0 in range(0, rows, 2048):    # |gpu - oracle| <= 1 BF16 ulp of the oracle value, in row chunks
        yo, yg = y_or[r0:r0 + 2048], y_gpu[r0:r0 + 2048]
        g = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        r = (yo.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        exp = ((yo >> 7) & 0xFF).astype(np.int64)
        ulp = np.ldexp(1.0, np.where(exp == 0, -126, exp - 127) - 7)
        within = within and bool(np.all(np.abs(g - r) <= ulp))
    ops = 2.0 * rows * w.N * w.K
    return {
        "value": round(ops / t / 1e12, 6),
        "unit": "TOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"leading {rows} of {w.M} rows, full N={w.N}, K={w.K} (rotate+quantize, exact INT32 GEMM, epilogue)"
                  + (" on unpacked INT4 codes" if int4 else ""),
        "seconds": round(t, 3),
        "sample_parity": {"rows": rows, "outputs": int(y_or.size), "not_bit_identical": int((~same).sum()),
                          "within_1_bf16_ulp": within},
    }


def calibrate_copy(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the clock settles over the first ~15 launches of the large GEMM (a kernel trace shows
    # its per-launch time falling from ~2.6-3.0 ms to ~2.33 ms), so the default warm-up
    # covers that before the timed region starts
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=3, help="workload id (synth.WORKLOADS)")
    ap.add_argument("--act", choices=["none", "gelu_tanh", "gelu_erf", "silu", "relu"], default="none",
                    help="input activation folded into the quantizer (int8_linear(input_act=...))")
    ap.add_argument("--fp6", action="store_true",
                    help="W4A4 workload on the FP6 matrix path (convrot_w4a4_linear_fp6)")
    ap.add_argument("--op", choices=["linear", "tensorwise", "attention"], default="linear",
                    help="linear: the whole layer (default); tensorwise: quantize_int8_tensorwise on the "
                         "workload's activations; attention: int8_attention on 40 heads x 16384 tokens x 128")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="row-major operands (int8_linear, convrot_w4a4_linear_fp6) instead of the K-sliced layout")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of BYTES bytes (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: the layer shards over rows or output channels without communication, "
              "so each GPU runs this same single-GPU step on its share.", flush=True)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return

    import numpy as np
    import torch

    import quantized_diffusion_amd as qd
    from synth import iter_w, iter_x, make_bias, workload

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    qd.lib()
    w = workload(args.workload)
    if args.op == "tensorwise":
        return bench_tensorwise(args, w)
    if args.op == "attention":
        return bench_attention(args)
    int4 = w.kind == "w4a4"
    act = ["none", "gelu_tanh", "gelu_erf", "silu", "relu"].index(args.act)
    if act and int4:
        sys.exit("an input activation is measured on the INT8 layer only")
    fp6 = args.fp6
    if fp6 and not int4:
        sys.exit("--fp6 applies to the W4A4 workload")
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name}: generating inputs")
    x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    for r0, r1, bits in iter_x(w):
        x[r0:r1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    Wf = torch.empty((N, K), dtype=torch.float32, device=dev)
    for r0, r1, chunk in iter_w(w):
        Wf[r0:r1].copy_(torch.from_numpy(chunk))
    b_bits = make_bias(w)
    bias = torch.from_numpy(b_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    # offline weight preparation (not timed)
    w_codes = None
    if fp6:
        wq, sw = qd.prepare_weights_w4a4_fp6(Wf)
        w_codes = qd.quantize_and_rotate_rowwise_int4(Wf)[0]    # the same codes, for the CPU baseline
    else:
        wq, sw = qd.prepare_weights_w4a4(Wf) if int4 else qd.prepare_weights(Wf)
    del Wf
    # weights in the K-sliced layout (also offline), unless asked for the row-major path:
    # INT8 weights, or the FP6 operand of the W4A4 layer
    sliced = not int4 and not args.row_major_weights and K % 64 == 0
    wsl = qd.slice_weights(wq) if sliced else None
    sliced6 = fp6 and not args.row_major_weights
    w6s = qd.fp6_slice_weights(wq, K) if sliced6 else None
    ws = torch.empty(qd.w4a4_fp6_workspace_size(M, K) if fp6 else qd.workspace_size(M, K), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # for the cold-cache steps below: allocated now, so that no allocation idles the GPU
    # between the timed sections
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        if sliced6:
            qd.convrot_w4a4_linear_fp6_sliced(x, w6s, sw, bias, 256, ws, y)
        elif fp6:
            qd.convrot_w4a4_linear_fp6(x, wq, sw, bias, 256, ws, y)
        elif int4:
            qd.convrot_w4a4_linear(x, wq, sw, bias, 256, ws, y)
        elif sliced:
            qd.int8_linear_sliced(x, wsl, sw, bias, act, 256, ws, y)
        elif act:
            qd.int8_linear_act(x, wq, sw, bias, act, 256, ws, y)
        else:
            qd.int8_linear(x, wq, sw, bias, 256, ws, y)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    ops = 2.0 * M * N * K
    tops = ops / (ms * 1e-3) / 1e12

    # distribution of single-step times (one event pair per step), then cold-cache steps: a
    # 512 MB scratch write before each (untimed) evicts the 256 MB Infinity Cache.  The
    # first 10 (fill, step) pairs are untimed, so the cold figure starts from the same
    # settled clock as the warm one.
    def timed_steps(n, before=None, skip=0):
        evs = []
        for i in range(skip + n):
            if before is not None:
                before()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            if i >= skip:
                evs.append((a, b))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    warm = timed_steps(args.steps)
    cold = timed_steps(min(args.steps, 10), lambda: scratch.fill_(1), skip=10)
    del scratch
    pick = lambda v, q: round(v[min(len(v) - 1, int(q * len(v)))], 5)
    step_times = {"warm_median": pick(warm, 0.5), "warm_min": round(warm[0], 5), "warm_p90": pick(warm, 0.9),
                  "cold_median": pick(cold, 0.5), "cold_min": round(cold[0], 5),
                  "note": "single steps timed with their own event pair; cold = after a 512 MB scratch write (10 untimed pairs first)"}

    # per-kernel durations (same kernels, launched through their own entry points)
    aq = torch.empty((M, K), dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    y2 = torch.empty_like(y)
    reps = max(5, args.steps)
    if sliced6:
        a6s = torch.empty((K // 128, M, 96), dtype=torch.uint8, device=dev)
        ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_fp6_sliced(x, 256, a6s, sx), reps, torch)
        ms_g = time_launches(lambda: qd.fp6_scaled_mm_sliced(a6s, sx, w6s, sw, bias, y2), reps, torch)
    elif fp6:
        a6 = torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=dev)
        ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_fp6(x, 256, a6, sx), reps, torch)
        ms_g = time_launches(lambda: qd.fp6_scaled_mm(a6, sx, wq, sw, K, bias, y2), reps, torch)
    elif int4:
        ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_int4(x, 256, aq, sx), reps, torch)
        ms_g = time_launches(lambda: qd.int4_scaled_mm(aq, sx, wq, sw, bias, y2), reps, torch)
    elif sliced:
        # the layer's own pair: K-sliced activation codes and weights
        asl = aq.view(K // 64, M, 64)
        ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_sliced(x, 256, asl, sx, act), reps, torch)
        ms_g = time_launches(lambda: qd.int8_scaled_mm_sliced(asl, sx, wsl, sw, bias, y2), reps, torch)
    else:
        if act:
            ms_q = time_launches(lambda: qd.quantize_rowwise_act(x, act, 256, aq, sx), reps, torch)
        else:
            ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise(x, 256, aq, sx), reps, torch)
        ms_g = time_launches(lambda: qd.int8_scaled_mm(aq, sx, wq, sw, bias, y2), reps, torch)
    same = bool(torch.equal(y2, y))
    q_bytes = (2.75 if fp6 else 3.0) * M * K + 4.0 * M
    g_min_bytes = float((M * K * 3 // 4 + N * K * 3 // 4) if fp6 else (M * K + (N * K // 2 if int4 else N * K))) \
        + 2 * M * N + 4 * M + 4 * N + 2 * N
    gemm_tops = ops / (ms_g * 1e-3) / 1e12
    traffic = load_traffic(w.name + (" (FP6, K-sliced)" if sliced6 else " (FP6)" if fp6 else
                                     " (row-major weights)" if not int4 and not sliced else ""))
    out = {
        "metric": (f"W4A4 rotated linear TOPS on the FP6 matrix path (incl. rotate+quant) & % of INT8 MFMA "
                   f"peak, M{M}/K{K}/N{N}" if fp6 else
                   f"W4A4 rotated linear TOPS (incl. rotate+quant) & % of INT8 MFMA peak, M{M}/K{K}/N{N}" if int4 else
                   f"INT8 linear TOPS with input_act={args.act} (incl. act+rotate+quant) & % of INT8 MFMA peak, "
                   f"M{M}/K{K}/N{N}" if act else
                   f"INT8 linear TOPS (incl. rotate+quant) & % of INT8 MFMA peak, M{M}/K{K}/N{N}"),
        "value": round(tops, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tops / (ops / (PAGE_MS[w.cid] * 1e-3) / 1e12), 4) if w.cid in PAGE_MS else None,
        "dtype": "i4 codes on fp6 (e2m3) MFMA" if fp6 else "i4 codes on i8 MFMA" if int4 else "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "input_act": args.act,
                   "rotation": "block-256 Walsh-Hadamard",
                   "activations": "bf16 -> int4 codes in int8 storage" if int4 else "bf16",
                   "weights": ("packed int4 per-channel fp32 scale, unpacked to int8 in the GEMM" if int4
                               else "int8 per-channel fp32 scale, K-sliced layout" if sliced
                               else "int8 per-channel fp32 scale, row-major"),
                   "bias": "bf16", "output": "bf16", "parallelism": "single GPU"},
        "frac_of_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
        "roofline": {"bound": "mfma", "kernel": ("gemm_f6_w8_kernel<MODE_BF16> (K-sliced operands)" if sliced6 else
                                                 "gemm_f6_w8_kernel<MODE_BF16>" if fp6 else
                                                 "gemm_i8_w8_kernel<MODE_BF16, 5, WF_I4>" if int4 else
                                                 "gemm_i8_w12_kernel<MODE_BF16> (256x384 tiles)"
                                                 if qd.int8_gemm_tiles(M, N, K) == qd.GEMM_TILES_256x384 else
                                                 "gemm_i8_w8_kernel<MODE_BF16, 4, WF_I8> (256x256 tiles)")
                     + (" (fused bf16 epilogue, K-sliced weights)" if sliced else " (fused bf16 epilogue)"),
                     "achieved": round(gemm_tops, 2), "peak": PEAK_FP6_TFLOPS if fp6 else PEAK_INT8_TOPS,
                     "unit": "TFLOP/s" if fp6 else "TOP/s",
                     "frac": round(gemm_tops / (PEAK_FP6_TFLOPS if fp6 else PEAK_INT8_TOPS), 4),
                     "traffic": traffic},
        "kernels": {
            "rotquant": {"ms": round(ms_q, 5), "algorithmic_bytes": q_bytes,
                         "GB_per_s": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
                         "frac_of_hbm": round(q_bytes / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "gemm": {"ms": round(ms_g, 5), "TOP_per_s": round(gemm_tops, 2),
                     "frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "min_hbm_bytes": g_min_bytes},
            "separate_launch_output_identical": same,
            "quantizer_writes": ("fp6 operand format, K-sliced" if sliced6 else "fp6 operand format" if fp6 else
                                 "int8 codes, K-sliced" if sliced else "int8 codes"),
        },
        "step_times_ms": step_times,
        "device": torch.cuda.get_device_name(0),
        "wall_s_timed_region": round(t_wall, 4),
        "context": "pages' figure for this workload: 10.5752 ms single call on an RTX 5090 D v2 (another machine)"
        if w.cid == 3 else None,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline(x, y, wq if w_codes is None else w_codes, sw, b_bits, w, torch,
                                           args.cpu_budget, act, codes=w_codes is not None)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_tensorwise(args, w):
    """quantize_int8_tensorwise on the workload's activation tensor: HBM-bound,
    algorithmic bytes 3MK + 4 (BF16 in, codes out, one scale)."""
    import numpy as np
    import torch

    import quantized_diffusion_amd as qd
    from synth import iter_x

    M, K = w.M, w.K
    dev = torch.device("cuda:0")
    log(f"[bench] tensorwise {w.name}: generating inputs")
    x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    for r0, r1, bits in iter_x(w):
        x[r0:r1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(qd.tensorwise_workspace_size(), dtype=torch.uint8, device=dev)

    def step():
        qd.quantize_int8_tensorwise(x, q, s, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_launches(step, args.steps, torch)
    alg = 3.0 * M * K + 4.0
    gbs = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": f"tensor-wise INT8 quantize GB/s (3MK+4 algorithmic bytes), M{M}/K{K}",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 -> i8", "data": "synthetic",
        "config": {"workload": w.name + " activations", "M": M, "K": K, "op": "quantize_int8_tensorwise",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "tw_amax_kernel + tw_quant_kernel (one step)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "note": "two passes over x: 5MK bytes move per step (x read twice)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        O = oracle.default()
        xh = x.view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        qo, so = O.quantize_tensorwise(xh, "bf16")
        t = time.perf_counter() - t0
        same = bool(np.array_equal(q.cpu().numpy(), qo)) and bool(s.cpu().numpy()[0] == so[0])
        out["cpu_baseline"] = {"value": round(alg / t / 1e9, 3), "unit": "GB/s", "cores": O.num_threads(),
                               "kind": "oracle", "sample": f"the whole {M}x{K} tensor", "seconds": round(t, 3),
                               "sample_parity": {"codes_and_scale_identical": same}}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_attention(args):
    """int8_attention (per-token quantization of q, k, v + the attention
    kernel) on BF16 q, k, v [40, 16384, 128]; 4 BH L^2 D operations per step."""
    import numpy as np
    import torch

    import quantized_diffusion_amd as qd

    BH, L, D = ATTN_BH, ATTN_L, ATTN_D
    dev = torch.device("cuda:0")
    log(f"[bench] int8_attention BH{BH}/L{L}/D{D}: generating inputs")
    gen = torch.Generator(device=dev).manual_seed(1234)
    q, k, v = (torch.randn((BH, L, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    ws = torch.empty(qd.attention_workspace_size(BH, L, L, D), dtype=torch.uint8, device=dev)
    y = torch.empty((BH, L, D), dtype=torch.bfloat16, device=dev)

    def step():
        qd.int8_attention(q, k, v, workspace=ws, out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_launches(step, args.steps, torch)
    t_wall = time.perf_counter() - t0
    al = lambda n: (n + 255) // 256 * 256
    offs = np.cumsum([0, al(BH * L * D), al(BH * L * D), al(BH * L * D), al(4 * BH * L), al(4 * BH * L)])
    qc, kc, vc = (ws[offs[i]:offs[i] + BH * L * D].view(BH, L, D).view(torch.int8) for i in range(3))
    sq, sk, sv = (ws[offs[3 + i]:offs[3 + i] + 4 * BH * L].view(torch.float32).view(BH, L) for i in range(3))
    y2 = torch.empty_like(y)
    ms_k = time_launches(lambda: qd.int8_attention_codes(qc, sq, kc, sk, vc, sv, out=y2), max(5, args.steps), torch)
    same = bool(torch.equal(y, y2))
    ops = 4.0 * BH * L * L * D
    tops = ops / (ms * 1e-3) / 1e12
    k_tops = ops / (ms_k * 1e-3) / 1e12
    out = {
        "metric": f"int8_attention TOPS (Q K^T on INT8, P V on BF16 matrix cores, incl. per-token quantization), "
                  f"BH{BH}/L{L}/D{D}",
        "value": round(tops, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 (scores), bf16 (probabilities x values)", "data": "synthetic",
        "config": {"workload": f"int8_attention BH{BH}/Lq{L}/Lk{L}/D{D}", "BH": BH, "Lq": L, "Lk": L, "D": D,
                   "inputs": "bf16 N(0,1)", "output": "bf16", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": f"attn_i8_kernel<{D}>", "achieved": round(k_tops, 2),
                     "peak": round(PEAK_ATTN_TOPS, 1), "unit": "TOP/s", "frac": round(k_tops / PEAK_ATTN_TOPS, 4),
                     "traffic": None,
                     "note": "peak = dense INT8 and BF16 matrix peaks combined for equal operation counts"},
        "kernels": {"attention": {"ms": round(ms_k, 5), "TOP_per_s": round(k_tops, 2)},
                    "quantizers": {"ms": round(ms - ms_k, 5)},
                    "codes_entry_output_identical": same},
        "device": torch.cuda.get_device_name(0),
        "wall_s_timed_region": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        O = oracle.default()
        h = lambda t: t.cpu().numpy()
        kch, skh, vch, svh = h(kc[:1]), h(sk[:1]), h(vc[:1]), h(sv[:1])
        n, t = 16, 0.0
        while True:       # grow the sample of head-0 queries until it takes a few seconds
            t0 = time.perf_counter()
            want = O.attention_codes(h(qc[:1, :n]), h(sq[:1, :n]), kch, skh, vch, svh)
            t = time.perf_counter() - t0
            if t > args.cpu_budget / 4 or n >= L:
                break
            n = min(L, n * 4)
        got = (y[:1, :n].contiguous().view(torch.int16).cpu().numpy().astype(np.uint32) << 16).view(np.float32)
        vmax = np.abs(svh[:, :, None].astype(np.float64) * vch).max(axis=1)
        bound = 2.0 ** -7 * vmax[:, None, :] + 2.0 ** -7 * np.abs(want)
        out["cpu_baseline"] = {"value": round(4.0 * n * L * D / t / 1e12, 6), "unit": "TOP/s",
                               "cores": O.num_threads(), "kind": "oracle",
                               "sample": f"{n} queries of head 0 against all {L} keys (float64 oracle on the codes)",
                               "seconds": round(t, 3),
                               "sample_parity": {"outputs": int(want.size),
                                                 "within_bound": bool(np.all(np.abs(got - want) <= bound))}}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
