#!/usr/bin/env python3
"""Benchmark of the rotated INT8 linear layer on one MI355X.

One step = one int8_linear call over the whole input (rotate+quantize kernel,
then the INT8 MFMA GEMM with the fused dequantizing epilogue), inputs already
resident in HBM.  The weights are prepared offline (rotated, quantized and
stored in the K-sliced layout: int8_linear_sliced; --row-major-weights runs
int8_linear on the row-major codes instead, same results).  The reported value is 2*M*N*K / step time in TOP/s (INT8
ops; the rotation and quantization are inside the timed step).

Prints ONE JSON line.  Besides the headline it carries:
  roofline        the GEMM kernel (dominant) against the dense INT8 MFMA peak
                  (published, and measured on this GPU), its duration measured
                  with HIP events on the launch stream;
  clock           the average shader clock over the timed steps (per-CU cycle
                  counters against the constant-rate wall counter, sampled on
                  the stream just before and after them);
  measured_peaks  this GPU's achievable dense INT8 matrix rate (random
                  operands changing every instruction) and HBM streaming
                  bandwidth (read, copy, and the quantizer's 2:1 mix);
  kernels         both kernels' average durations, TOP/s or GB/s and fractions;
  per_config      the other large workloads (odd M, wide MLP, W4A4 on the FP6
                  path) measured in the same run: ms, TOP/s, fractions, and
                  in their own cpu_baseline leg a sampled comparison with the
                  oracle;
  cpu_baseline    the plain C oracle timed on the host cores over a bounded
                  sample of the same workload (the leading rows), rotate+quant
                  and GEMM+epilogue timed separately, and the GPU output of
                  those rows compared with it.
The oracle is used only by the cpu_baseline legs (outside every timed
region; --no-cpu-baseline skips them all).

Usage: python bench.py [--gpus 1] [--steps 30] [--warmup 30] [--workload 3]
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


MEASURE_LIB = os.path.join(ROOT, "quantized_diffusion_amd", "libqdmeasure.so")
SPEC_CLOCK_MHZ = 2400.0      # MI355X peak engine clock: the published peaks are quoted at it
PER_CONFIG = (2, 4, 5)       # large workloads measured beside the headline (5 on the FP6 path)


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


# ------------------------------------------------------------------ machine measurements

_mlib = None


def measure_lib():
    """libqdmeasure.so: the benchmark's measurement kernels (matrix-core and
    streaming probes, clock samples), built beside the layer's library."""
    global _mlib
    if _mlib is None:
        import ctypes
        if not os.path.exists(MEASURE_LIB):
            raise ImportError(f"{MEASURE_LIB} not found: build it with `python -m quantized_diffusion_amd.build`")
        L = ctypes.CDLL(MEASURE_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qdm_mfma_i8.argtypes = [P, I64, I, I, P, P]
        L.qdm_read.argtypes = [P, I64, I, P, P]
        L.qdm_copy.argtypes = [P, P, I64, I, P]
        L.qdm_mix21.argtypes = [P, P, I64, I, P]
        L.qdm_clock_sample.argtypes = [P, I, P]
        _mlib = L
    return _mlib


def _vp(t):
    import ctypes
    return ctypes.c_void_p(t.data_ptr())


def _cur_stream(torch):
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _mcheck(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: launch failed (HIP error {rc})")


def per_cu_clock(samples, rate_khz: float):
    """samples [2, B, 4] int64 (cycle counter, wall counter, XCD, HW_ID) taken
    before and after a region -> the average shader clock (MHz) per compute unit.
    Cycle counters of different compute units are not aligned with one another,
    so each CU is timed from its own earliest sample before to its own latest
    sample after.  Returns {(xcd, cu id bits): MHz}."""
    def pick(rows, last):
        d = {}
        for c, w, x, h in rows:
            key = (int(x), (int(h) >> 8) & 0xFF)     # XCD; engine, array and CU fields of HW_ID
            if key not in d or ((w > d[key][1]) if last else (w < d[key][1])):
                d[key] = (int(c), int(w))
        return d
    d0, d1 = pick(samples[0], False), pick(samples[1], True)
    out = {}
    for k in set(d0) & set(d1):
        dw = d1[k][1] - d0[k][1]
        if dw > 0:
            out[k] = (d1[k][0] - d0[k][0]) / (dw / rate_khz) / 1e3
    return out


class ClockProbe:
    """Average shader clock over a region of the current stream: a kernel of
    4096 one-wave workgroups samples every compute unit's cycle counter and the
    constant-rate wall counter just before and just after the region."""
    BLOCKS = 4096

    def __init__(self, torch):
        self.torch = torch
        self.L = measure_lib()
        self.rate_khz = float(self.L.qdm_wall_clock_khz())
        self.buf = torch.zeros((2, self.BLOCKS, 4), dtype=torch.int64, device="cuda")

    def _sample(self, i):
        _mcheck(self.L.qdm_clock_sample(_vp(self.buf[i]), self.BLOCKS, _cur_stream(self.torch)), "clock sample")

    def start(self):
        self._sample(0)

    def stop(self):
        self._sample(1)

    def result(self):
        """After a synchronize: median clock over the compute units, per XCD."""
        import numpy as np
        if self.rate_khz <= 0:
            return None
        cu = per_cu_clock(self.buf.cpu().numpy(), self.rate_khz)
        if not cu:
            return None
        mhz = np.array(list(cu.values()))
        xcd = np.array([k[0] for k in cu])
        return {"avg_mhz": round(float(np.median(mhz)), 1),
                "per_xcd_mhz": [round(float(np.median(mhz[xcd == x])), 1) for x in sorted(set(xcd.tolist()))],
                "compute_units": int(mhz.size),
                "method": "per-CU shader cycle counter against the 100 MHz wall counter, sampled on the stream "
                          "just before and after the region; median over CUs"}


def measured_peaks(torch):
    """This GPU's achievable dense INT8 matrix-core rate (eight accumulator
    chains per wave, random operands changing on every instruction, two waves
    per SIMD on every CU) and its HBM streaming bandwidth: read only, copy, and
    two bytes read per byte written (the quantizer's mix); 16-byte
    non-temporal accesses, 32768 workgroups, 2 GiB of input."""
    L = measure_lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    src = torch.randint(-128, 128, (1 << 20,), dtype=torch.int8, device=dev, generator=g)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    blocks, iters = 1024, 200
    ops = blocks * 4.0 * iters * 64 * 65536
    mfma = lambda: _mcheck(L.qdm_mfma_i8(_vp(src), src.numel() // 16, blocks, iters, _vp(sink), _cur_stream(torch)),
                           "matrix-core probe")
    for _ in range(20):                 # the clock settles under the load first
        mfma()
    torch.cuda.synchronize()
    clk = ClockProbe(torch)
    n = 40
    clk.start()
    ms = time_launches(mfma, n, torch)
    clk.stop()
    torch.cuda.synchronize()
    c = clk.result()
    tops = ops / (ms * 1e-3) / 1e12
    out = {"int8_mfma": {"TOP_per_s": round(tops, 1), "frac_of_spec": round(tops / PEAK_INT8_TOPS, 4),
                         "clock_mhz": c["avg_mhz"] if c else None,
                         "frac_of_spec_at_that_clock": round(tops / (PEAK_INT8_TOPS * c["avg_mhz"] / SPEC_CLOCK_MHZ), 4)
                         if c else None,
                         "probe": f"v_mfma_i32_32x32x32_i8, {blocks} workgroups x 4 waves x {iters * 64} "
                                  "instructions, operands from random bytes, rotated every instruction"}}
    del src
    nb = 2 << 30
    a = torch.empty(nb, dtype=torch.uint8, device=dev)
    a.random_(generator=g)
    b = torch.empty(nb // 2, dtype=torch.uint8, device=dev)
    SB = 32768
    s = lambda: _cur_stream(torch)
    probes = (("read", lambda: L.qdm_read(_vp(a), nb, SB, _vp(sink), s()), nb),
              ("copy", lambda: L.qdm_copy(_vp(a), _vp(b), nb // 2, SB, s()), nb),
              ("read2_write1", lambda: L.qdm_mix21(_vp(a), _vp(b), nb // 2, SB, s()), nb + nb // 2))
    hbm = {}
    for name, fn, nbytes in probes:
        f = lambda: _mcheck(fn(), f"{name} probe")
        ms = time_launches(f, 5, torch)
        gbs = nbytes / (ms * 1e-3) / 1e9
        hbm[name] = {"GB_per_s": round(gbs, 1), "frac_of_spec": round(gbs / PEAK_HBM_GBS, 4)}
    out["hbm"] = hbm
    del a, b
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ the layer

class LinearRun:
    """One workload of the layer on the GPU: inputs, offline weights, the step
    and its two kernels launched through their own entry points."""

    def __init__(self, w, torch, fp6=False, act=0, row_major=False, keep_host=False):
        import numpy as np

        import quantized_diffusion_amd as qd
        from synth import iter_w, iter_x, make_bias
        self.w, self.torch, self.qd = w, torch, qd
        self.int4 = w.kind == "w4a4"
        self.fp6, self.act = fp6, act
        if act and self.int4:
            raise ValueError("an input activation is measured on the INT8 layer only")
        if fp6 and not self.int4:
            raise ValueError("the FP6 path applies to the W4A4 workload")
        M, K, N = self.M, self.K, self.N = w.M, w.K, w.N
        dev = torch.device("cuda:0")
        log(f"[bench] {w.name}: generating inputs")
        self.x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        for r0, r1, bits in iter_x(w):
            self.x[r0:r1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
        Wf = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.W_host = np.empty((N, K), np.float32) if keep_host else None
        for r0, r1, chunk in iter_w(w):
            Wf[r0:r1].copy_(torch.from_numpy(chunk))
            if keep_host:
                self.W_host[r0:r1] = chunk
        self.b_bits = make_bias(w)
        self.bias = torch.from_numpy(self.b_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        # offline weight preparation (not timed)
        self.w_codes = None
        if fp6:
            self.wq, self.sw = qd.prepare_weights_w4a4_fp6(Wf)
            self.w_codes = qd.quantize_and_rotate_rowwise_int4(Wf)[0]   # the same codes, for the CPU baseline
        else:
            self.wq, self.sw = qd.prepare_weights_w4a4(Wf) if self.int4 else qd.prepare_weights(Wf)
        del Wf
        # weights in the K-sliced layout (also offline), unless asked for the row-major path
        self.sliced = not self.int4 and not row_major and K % 64 == 0
        self.wsl = qd.slice_weights(self.wq) if self.sliced else None
        self.sliced6 = fp6 and not row_major
        self.w6s = qd.fp6_slice_weights(self.wq, K) if self.sliced6 else None
        self.ws = torch.empty(qd.w4a4_fp6_workspace_size(M, K) if fp6 else qd.workspace_size(M, K),
                              dtype=torch.uint8, device=dev)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

    def step(self):
        qd, x, sw, bias, ws, y = self.qd, self.x, self.sw, self.bias, self.ws, self.y
        if self.sliced6:
            qd.convrot_w4a4_linear_fp6_sliced(x, self.w6s, sw, bias, 256, ws, y)
        elif self.fp6:
            qd.convrot_w4a4_linear_fp6(x, self.wq, sw, bias, 256, ws, y)
        elif self.int4:
            qd.convrot_w4a4_linear(x, self.wq, sw, bias, 256, ws, y)
        elif self.sliced:
            qd.int8_linear_sliced(x, self.wsl, sw, bias, self.act, 256, ws, y)
        elif self.act:
            qd.int8_linear_act(x, self.wq, sw, bias, self.act, 256, ws, y)
        else:
            qd.int8_linear(x, self.wq, sw, bias, 256, ws, y)

    @property
    def ops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def kernel_name(self) -> str:
        qd = self.qd
        name = ("gemm_f6_w4_kernel<MODE_BF16> (K-sliced operands)" if self.sliced6 else
                "gemm_f6_w4_kernel<MODE_BF16>" if self.fp6 else
                "gemm_i8_w8_kernel<MODE_BF16, 5, WF_I4>" if self.int4 else
                "gemm_i8_w12_kernel<MODE_BF16> (256x384 tiles)"
                if qd.int8_gemm_tiles(self.M, self.N, self.K) == qd.GEMM_TILES_256x384 else
                "gemm_i8_w8_kernel<MODE_BF16, 4, WF_I8> (256x256 tiles)")
        return name + (" (fused bf16 epilogue, K-sliced weights)" if self.sliced else " (fused bf16 epilogue)")

    def time_kernels(self, reps: int):
        """(quantizer ms, GEMM ms, GEMM output identical to the step's): the step's
        two kernels launched through their own entry points, back to back."""
        torch, qd, M, K = self.torch, self.qd, self.M, self.K
        x, sw, bias = self.x, self.sw, self.bias
        dev = x.device
        aq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        y2 = torch.empty_like(self.y)
        if self.sliced6:
            a6s = torch.empty((K // 128, M, 96), dtype=torch.uint8, device=dev)
            ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_fp6_sliced(x, 256, a6s, sx), reps, torch)
            ms_g = time_launches(lambda: qd.fp6_scaled_mm_sliced(a6s, sx, self.w6s, sw, bias, y2), reps, torch)
        elif self.fp6:
            a6 = torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=dev)
            ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_fp6(x, 256, a6, sx), reps, torch)
            ms_g = time_launches(lambda: qd.fp6_scaled_mm(a6, sx, self.wq, sw, K, bias, y2), reps, torch)
        elif self.int4:
            ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_int4(x, 256, aq, sx), reps, torch)
            ms_g = time_launches(lambda: qd.int4_scaled_mm(aq, sx, self.wq, sw, bias, y2), reps, torch)
        elif self.sliced:
            # the layer's own pair: K-sliced activation codes and weights
            asl = aq.view(K // 64, M, 64)
            ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise_sliced(x, 256, asl, sx, self.act), reps, torch)
            ms_g = time_launches(lambda: qd.int8_scaled_mm_sliced(asl, sx, self.wsl, sw, bias, y2), reps, torch)
        else:
            if self.act:
                ms_q = time_launches(lambda: qd.quantize_rowwise_act(x, self.act, 256, aq, sx), reps, torch)
            else:
                ms_q = time_launches(lambda: qd.quantize_and_rotate_rowwise(x, 256, aq, sx), reps, torch)
            ms_g = time_launches(lambda: qd.int8_scaled_mm(aq, sx, self.wq, sw, bias, y2), reps, torch)
        same = bool(torch.equal(y2, self.y))
        return ms_q, ms_g, same

    def quant_bytes(self) -> float:
        return (2.75 if self.fp6 else 3.0) * self.M * self.K + 4.0 * self.M

    def gemm_min_bytes(self) -> float:
        M, K, N = self.M, self.K, self.N
        operands = (M * K * 3 // 4 + N * K * 3 // 4) if self.fp6 else (M * K + (N * K // 2 if self.int4 else N * K))
        return float(operands) + 2 * M * N + 4 * M + 4 * N + 2 * N

    def gemm_peak(self) -> float:
        return PEAK_FP6_TFLOPS if self.fp6 else PEAK_INT8_TOPS

    def sampled_parity(self, O, n: int = 4000, seed: int = 9100):
        """n random outputs plus the whole last row against the oracle (its own
        weight preparation from the FP32 weights, its quantizer on the sampled
        rows, then the exact dot products and the epilogue at each point)."""
        import numpy as np
        torch, w = self.torch, self.w
        qmax = 7 if self.int4 else 127
        wq_o, sw_o = O.prepare_weights(self.W_host, 256, qmax=qmax)
        g = np.random.Generator(np.random.PCG64(seed + w.cid))
        rows = np.concatenate([g.integers(0, self.M, n), np.full(self.N, self.M - 1)])
        cols = np.concatenate([g.integers(0, self.N, n), np.arange(self.N)])
        urows, inv = np.unique(rows, return_inverse=True)
        xr = self.x[torch.from_numpy(urows).to(self.x.device)].contiguous()
        x_host = xr.view(torch.int16).cpu().numpy().view(np.uint16)
        qo, so = O.quantize_rowwise(x_host, "bf16", 256, qmax=qmax, act=self.act)
        yo, _ = O.linear_points(qo, so, inv, wq_o, sw_o, self.b_bits, cols)
        dev = self.y.device
        yg = self.y[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)]
        yg = yg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        same = yg == yo
        gf = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rf = (yo.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        exp = ((yo >> 7) & 0xFF).astype(np.int64)
        ulp = np.ldexp(1.0, np.where(exp == 0, -126, exp - 127) - 7)
        return {"outputs": int(yo.size), "not_bit_identical": int((~same).sum()),
                "within_1_bf16_ulp": bool(np.all(np.abs(gf - rf) <= ulp))}


def time_steps(run, steps: int, warmup: int, torch, clock: bool = True):
    """warmup untimed steps, then `steps` steps between one pair of HIP events
    (and the clock samples just outside them): (ms per step, wall s, clock)."""
    # everything the timed region needs is allocated before the warm-up: an
    # allocation (or any idle gap) between warm-up and timing would restart the
    # clock's settling transient (the first launches after idle run slower)
    clk = ClockProbe(torch) if clock else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if clk:
        clk.start()
    e0.record()
    for _ in range(steps):
        run.step()
    e1.record()
    if clk:
        clk.stop()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return e0.elapsed_time(e1) / steps, t_wall, (clk.result() if clk else None)


def measure_config(cid: int, args, torch, O):
    """One of the other large workloads, measured in the same run as the headline."""
    from synth import workload
    w = workload(cid)
    fp6 = w.kind == "w4a4"
    run = LinearRun(w, torch, fp6=fp6, keep_host=O is not None)
    ms, _, clk = time_steps(run, max(10, args.steps), args.warmup, torch)
    ms_q, ms_g, same = run.time_kernels(max(5, args.steps))
    g_tops = run.ops / (ms_g * 1e-3) / 1e12
    q_gbs = run.quant_bytes() / (ms_q * 1e-3) / 1e9
    out = {"workload": w.name, "M": w.M, "K": w.K, "N": w.N,
           "path": "convrot_w4a4_linear_fp6_sliced (INT4 codes on FP6 MFMA)" if fp6 else "int8_linear_sliced",
           "ms_per_step": round(ms, 5), "TOP_per_s": round(run.ops / (ms * 1e-3) / 1e12, 2),
           "frac_of_int8_peak": round(run.ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
           "gemm": {"kernel": run.kernel_name(), "ms": round(ms_g, 5), "TOP_per_s": round(g_tops, 2),
                    "peak": run.gemm_peak(), "frac": round(g_tops / run.gemm_peak(), 4)},
           "rotquant": {"ms": round(ms_q, 5), "GB_per_s": round(q_gbs, 1), "frac_of_hbm": round(q_gbs / PEAK_HBM_GBS, 4)},
           "separate_launch_output_identical": same, "clock": clk}
    if w.cid in PAGE_MS:
        out["context_page_ms"] = PAGE_MS[w.cid]
    if O is not None:   # the cpu_baseline leg of this line: its oracle checks sampled outputs
        log(f"[bench] {w.name}: cpu baseline leg, sampled outputs against the oracle")
        out["cpu_baseline"] = {"kind": "oracle", "sample": "4000 random outputs and the whole last row",
                               "sampled_parity": run.sampled_parity(O)}
    del run
    torch.cuda.empty_cache()
    return out


def cpu_baseline(run, torch, budget_s: float):
    """Time the oracle on the leading rows of the same workload, rotate+quant and
    GEMM+epilogue separately; check those rows of the GPU output against it."""
    import numpy as np

    import oracle
    O = oracle.default()
    w, int4, act = run.w, run.int4, run.act
    qmax = 7 if int4 else 127
    wq = (run.wq if run.w_codes is None else run.w_codes).cpu().numpy()
    if int4 and run.w_codes is None:
        wq = O.unpack_int4(wq, w.K)     # packed weights -> INT4 codes in INT8 storage
    sw = run.sw.cpu().numpy()

    def halves(rows):
        x = run.x[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        q, s = O.quantize_rowwise(x, "bf16", 256, qmax=qmax, act=act)
        t1 = time.perf_counter()
        y = O.epilogue(O.gemm_i32(q, wq), s, sw, run.b_bits)
        return t1 - t0, time.perf_counter() - t1, y

    tq, tg, _ = halves(16)
    rows = int(min(w.M, max(16, 16 * budget_s / max(tq + tg, 1e-3))))
    rows = min(rows, 20000)       # about 10-15 s of oracle work on the host's cores
    tq, tg, y_or = halves(rows)
    y_gpu = run.y[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
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
    q_bytes = 3.0 * rows * w.K + 4.0 * rows
    return {
        "value": round(ops / (tq + tg) / 1e12, 6),
        "unit": "TOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"leading {rows} of {w.M} rows, full N={w.N}, K={w.K} (rotate+quantize, exact INT32 GEMM, epilogue)"
                  + (" on unpacked INT4 codes" if int4 else ""),
        "seconds": round(tq + tg, 3),
        "rotate_quant": {"seconds": round(tq, 3), "GB_per_s": round(q_bytes / tq / 1e9, 3)},
        "gemm_epilogue": {"seconds": round(tg, 3), "TOP_per_s": round(ops / tg / 1e12, 6)},
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
    ap.add_argument("--op", choices=["linear", "tensorwise", "attention", "peaks"], default="linear",
                    help="linear: the whole layer (default); tensorwise: quantize_int8_tensorwise on the "
                         "workload's activations; attention: int8_attention on 40 heads x 16384 tokens x 128; "
                         "peaks: only this GPU's measured matrix-core and HBM ceilings")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="row-major operands (int8_linear, convrot_w4a4_linear_fp6) instead of the K-sliced layout")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="skip the other large workloads")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured matrix-core and HBM ceilings")
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

    import torch

    import quantized_diffusion_amd as qd
    from synth import workload

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    qd.lib()
    w = workload(args.workload)
    if args.op == "peaks":
        print(json.dumps({"measured_peaks": measured_peaks(torch), "device": torch.cuda.get_device_name(0)}),
              flush=True)
        return
    if args.op == "tensorwise":
        return bench_tensorwise(args, w)
    if args.op == "attention":
        return bench_attention(args)
    act = ["none", "gelu_tanh", "gelu_erf", "silu", "relu"].index(args.act)
    if act and w.kind == "w4a4":
        sys.exit("an input activation is measured on the INT8 layer only")
    if args.fp6 and w.kind != "w4a4":
        sys.exit("--fp6 applies to the W4A4 workload")
    run = LinearRun(w, torch, fp6=args.fp6, act=act, row_major=args.row_major_weights)
    M, K, N = w.M, w.K, w.N
    # for the cold-cache steps below: allocated now, so that no allocation idles the GPU
    # between the timed sections
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    ms, t_wall, clock = time_steps(run, args.steps, args.warmup, torch)
    ops = run.ops
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
            run.step()
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
    ms_q, ms_g, same = run.time_kernels(max(5, args.steps))
    fp6, int4, sliced, sliced6 = run.fp6, run.int4, run.sliced, run.sliced6
    q_bytes = run.quant_bytes()
    gemm_tops = ops / (ms_g * 1e-3) / 1e12
    peak = run.gemm_peak()
    traffic = load_traffic(w.name + (" (FP6, K-sliced)" if sliced6 else " (FP6)" if fp6 else
                                     " (row-major weights)" if not int4 and not sliced else ""))
    peaks = None
    if not args.no_peaks:
        log("[bench] measured matrix-core and HBM ceilings")
        peaks = measured_peaks(torch)
    q_gbs = q_bytes / (ms_q * 1e-3) / 1e9
    roofline = {"bound": "mfma", "kernel": run.kernel_name(), "achieved": round(gemm_tops, 2), "peak": peak,
                "unit": "TFLOP/s" if fp6 else "TOP/s", "frac": round(gemm_tops / peak, 4), "traffic": traffic}
    if peaks and not fp6:
        mp = peaks["int8_mfma"]["TOP_per_s"]
        roofline["measured_peak"] = mp
        roofline["frac_of_measured_peak"] = round(gemm_tops / mp, 4)
    if clock and clock.get("avg_mhz"):
        roofline["frac_of_peak_at_step_clock"] = round(gemm_tops / (peak * clock["avg_mhz"] / SPEC_CLOCK_MHZ), 4)
    rotquant = {"ms": round(ms_q, 5), "algorithmic_bytes": q_bytes, "GB_per_s": round(q_gbs, 1),
                "frac_of_hbm": round(q_gbs / PEAK_HBM_GBS, 4)}
    if peaks:
        mix = peaks["hbm"]["read2_write1"]["GB_per_s"]
        rotquant["measured_read2_write1_GB_per_s"] = mix
        rotquant["frac_of_measured_read2_write1"] = round(q_gbs / mix, 4)
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
        "roofline": roofline,
        "clock": clock,
        "kernels": {
            "rotquant": rotquant,
            "gemm": {"ms": round(ms_g, 5), "TOP_per_s": round(gemm_tops, 2),
                     "frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "min_hbm_bytes": run.gemm_min_bytes()},
            "separate_launch_output_identical": same,
            "quantizer_writes": ("fp6 operand format, K-sliced" if sliced6 else "fp6 operand format" if fp6 else
                                 "int8 codes, K-sliced" if sliced else "int8 codes"),
        },
        "measured_peaks": peaks,
        "step_times_ms": step_times,
        "device": torch.cuda.get_device_name(0),
        "wall_s_timed_region": round(t_wall, 4),
        "context": "pages' figure for this workload: 10.5752 ms single call on an RTX 5090 D v2 (another machine)"
        if w.cid == 3 else None,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline(run, torch, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    if not args.no_per_config and w.cid == 3 and not act and not args.row_major_weights:
        del run
        torch.cuda.empty_cache()
        O = None
        if not args.no_cpu_baseline:
            import oracle
            O = oracle.default()
        out["per_config"] = [measure_config(c, args, torch, O) for c in PER_CONFIG]
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
        # the parity bound of the GPU tests (rounding steps of the kernel, evaluated with the
        # oracle's softmax probabilities)
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from attention_bound import attention_bound
        qch, sqh = h(qc[:1, :n]), h(sq[:1, :n])
        P = O.attention_probs(qch, sqh, kch, skh)
        bound = attention_bound(want, P, qch, sqh, kch, skh, vch, svh, 1.0 / np.sqrt(D))
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
