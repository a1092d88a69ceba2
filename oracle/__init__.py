"""Oracle for the rotated, dynamically quantized INT8/INT4 linear layer (and INT8 attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never calls it and shares no code with it; the GPU library fails loudly when
its own HIP extension is missing instead of falling back to anything here.

The arithmetic lives in ``qdiff_oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``, no fast-math); this module is ctypes marshalling over
NumPy arrays.  The header of the C file lists the passages of the pages each
step follows and the readings taken where they are silent.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force with exact rationals / Python
integers, closed forms, invariants, error bounds); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "qdiff_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "f16": F16}

CFLAGS = ["-O3", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-march=x86-64-v3", "-Wall", "-Wextra"]


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    return compile_source(SRC_PATH, LIB_PATH, verbose)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bind(L):
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_attention_i8.restype = None
    L.oracle_attention_i8.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_double, P]
    L.oracle_attention_probs.restype = None
    L.oracle_attention_probs.argtypes = [P, P, P, P, I64, I64, I64, I64, ctypes.c_double, P]
    L.oracle_bf16_rne.restype = ctypes.c_uint16
    L.oracle_bf16_rne.argtypes = [ctypes.c_float]
    L.oracle_hadamard256.argtypes = [P]
    L.oracle_rotate_rows.restype = I
    L.oracle_rotate_rows.argtypes = [P, I, I64, I64, I64, I, P]
    L.oracle_quantize_rows.argtypes = [P, I64, I64, I, P, I64, P]
    L.oracle_quantize_rowwise.restype = I
    L.oracle_quantize_rowwise.argtypes = [P, I, I64, I64, I64, I, I, P, I64, P]
    L.oracle_quantize_tensorwise.restype = I
    L.oracle_quantize_tensorwise.argtypes = [P, I, I64, I64, I64, I, P, I64, P]
    L.oracle_gemm_i32.restype = I64
    L.oracle_gemm_i32.argtypes = [P, I64, I64, I64, P, I64, I64, P]
    L.oracle_epilogue.argtypes = [P, I64, I64, P, P, P, P]
    L.oracle_epilogue_f32.argtypes = [P, I64, I64, P, P, P, P]
    L.oracle_linear_act.restype = I
    L.oracle_linear_act.argtypes = [P, I, I64, I64, I64, I, P, P, P, I64, I, I, P]
    L.oracle_quantize_rowwise_act.restype = I
    L.oracle_quantize_rowwise_act.argtypes = [P, I, I64, I64, I64, I, I, I, P, I64, P]
    L.oracle_input_act.argtypes = [P, I, I64, I, P]
    L.oracle_linear.restype = I
    L.oracle_linear.argtypes = [P, I, I64, I64, I64, P, P, P, I64, I, I, P]
    L.oracle_linear_points.argtypes = [P, I64, P, P, P, P, P, P, I64, P, P]
    L.oracle_dequantize.argtypes = [P, I64, I64, I64, P, I, I, P]
    L.oracle_pack_int4.argtypes = [P, I64, I64, P]
    L.oracle_unpack_int4.argtypes = [P, I64, I64, P]
    L.oracle_bf16_rne_array.argtypes = [P, I64, P]
    L.oracle_num_threads.restype = I
    return L


def _x_in(x: np.ndarray, dtype: str) -> np.ndarray:
    want = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[dtype]
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be a {np.dtype(want).name} array, got {x.dtype}")
    return np.ascontiguousarray(x)


class Oracle:
    """ctypes view of one compiled copy of ``qdiff_oracle.c``."""

    def __init__(self, lib_path: str = LIB_PATH):
        self.L = _bind(ctypes.CDLL(lib_path))

    def num_threads(self) -> int:
        return self.L.oracle_num_threads()

    def bf16_rne(self, f) -> np.ndarray:
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.shape, np.uint16)
        self.L.oracle_bf16_rne_array(_p(f), f.size, _p(out))
        return out

    def hadamard256(self, u) -> np.ndarray:
        """Rotated copy of one 256-element FP32 block."""
        v = np.array(u, dtype=np.float32, copy=True).reshape(256)
        self.L.oracle_hadamard256(_p(v))
        return v

    def rotate_rows(self, x, dtype: str = "bf16", block: int = 256) -> np.ndarray:
        """FP32 rows of x, each 256-block rotated when block == 256."""
        x = _x_in(x, dtype)
        M, K = x.shape
        out = np.empty((M, K), np.float32)
        if self.L.oracle_rotate_rows(_p(x), _DTYPES[dtype], M, K, K, block, _p(out)):
            raise ValueError(f"oracle_rotate_rows: unsupported block={block} / K={K}")
        return out

    def quantize_rows(self, v, qmax: int = 127):
        """Per-row symmetric quantization of FP32 rows (no rotation)."""
        v = np.ascontiguousarray(v, dtype=np.float32)
        M, K = v.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        self.L.oracle_quantize_rows(_p(v), M, K, qmax, _p(q), K, _p(s))
        return q, s

    def quantize_rowwise(self, x, dtype: str = "bf16", block: int = 256, qmax: int = 127, act: int = 0):
        """(codes int8 [M, K], row scales float32 [M]) of [activation,] rotate-then-quantize."""
        x = _x_in(x, dtype)
        M, K = x.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        if act:
            rc = self.L.oracle_quantize_rowwise_act(_p(x), _DTYPES[dtype], M, K, K, block, act, qmax, _p(q), K,
                                                    _p(s))
        else:
            rc = self.L.oracle_quantize_rowwise(_p(x), _DTYPES[dtype], M, K, K, block, qmax, _p(q), K, _p(s))
        if rc:
            raise ValueError(f"oracle_quantize_rowwise failed rc={rc}")
        return q, s

    def quantize_tensorwise(self, x, dtype: str = "bf16", qmax: int = 127):
        """(codes int8 [M, K], scale float32 [1]) of tensor-wise quantization (no rotation)."""
        x = _x_in(x, dtype)
        M, K = x.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(1, np.float32)
        self.L.oracle_quantize_tensorwise(_p(x), _DTYPES[dtype], M, K, K, qmax, _p(q), K, _p(s))
        return q, s

    def prepare_weights(self, w, block: int = 256, qmax: int = 127):
        """Offline weight preparation: rotate FP32 W [N, K] along K, quantize per output channel."""
        return self.quantize_rowwise(np.ascontiguousarray(w, dtype=np.float32), "f32", block, qmax)

    def gemm_i32(self, a, w) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.int8)
        w = np.ascontiguousarray(w, dtype=np.int8)
        M, K = a.shape
        N, K2 = w.shape
        if K != K2:
            raise ValueError("K mismatch")
        acc = np.empty((M, N), np.int32)
        bad = self.L.oracle_gemm_i32(_p(a), M, K, K, _p(w), N, K, _p(acc))
        if bad:
            raise OverflowError(f"{bad} accumulators do not fit in int32")
        return acc

    def _epi_args(self, acc, sx, sw, bias):
        acc = np.ascontiguousarray(acc, dtype=np.int32)
        sx = np.ascontiguousarray(sx, dtype=np.float32)
        sw = np.ascontiguousarray(sw, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        return acc, sx, sw, b

    def epilogue(self, acc, sx, sw, bias=None) -> np.ndarray:
        acc, sx, sw, b = self._epi_args(acc, sx, sw, bias)
        M, N = acc.shape
        y = np.empty((M, N), np.uint16)
        self.L.oracle_epilogue(_p(acc), M, N, _p(sx), _p(sw), _p(b), _p(y))
        return y

    def epilogue_f32(self, acc, sx, sw, bias=None) -> np.ndarray:
        acc, sx, sw, b = self._epi_args(acc, sx, sw, bias)
        M, N = acc.shape
        t = np.empty((M, N), np.float32)
        self.L.oracle_epilogue_f32(_p(acc), M, N, _p(sx), _p(sw), _p(b), _p(t))
        return t

    def input_act(self, x, dtype: str, act: int) -> np.ndarray:
        """act(x) elementwise, rounded to the 16-bit input type; uint16 bits."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        out = np.empty_like(x)
        self.L.oracle_input_act(_p(x), _DTYPES[dtype], x.size, act, _p(out))
        return out

    def linear(self, x, wq, sw, bias=None, dtype: str = "bf16", block: int = 256,
               qmax: int = 127, act: int = 0) -> np.ndarray:
        """The whole layer: BF16 output bits [M, N]."""
        x = _x_in(x, dtype)
        M, K = x.shape
        wq = np.ascontiguousarray(wq, dtype=np.int8)
        N = wq.shape[0]
        sw = np.ascontiguousarray(sw, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        y = np.empty((M, N), np.uint16)
        rc = self.L.oracle_linear_act(_p(x), _DTYPES[dtype], M, K, K, act, _p(wq), _p(sw), _p(b), N,
                                  block, qmax, _p(y))
        if rc:
            raise RuntimeError(f"oracle_linear failed rc={rc}")
        return y

    def linear_points(self, aq, sx, aq_rows, wq, sw, bias, cols):
        """(y bits, acc) at points (aq_rows[i], cols[i]) from activation codes aq."""
        aq = np.ascontiguousarray(aq, dtype=np.int8)
        K = aq.shape[1]
        sx = np.ascontiguousarray(sx, dtype=np.float32)
        aq_rows = np.ascontiguousarray(aq_rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        wq = np.ascontiguousarray(wq, dtype=np.int8)
        sw = np.ascontiguousarray(sw, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        n = cols.size
        y = np.empty(n, np.uint16)
        acc = np.empty(n, np.int32)
        self.L.oracle_linear_points(_p(aq), K, _p(sx), _p(aq_rows), _p(wq), _p(sw), _p(b),
                                    _p(cols), n, _p(y), _p(acc))
        return y, acc

    def attention_codes(self, qc, sq, kc, sk, vc, sv, scale=None) -> np.ndarray:
        """INT8 attention on per-token codes: qc [BH, Lq, D], kc / vc [BH, Lk, D],
        scales [BH, L]; float64 [BH, Lq, D] (the reading in qdiff_oracle.c)."""
        qc, kc, vc = (np.ascontiguousarray(a, dtype=np.int8) for a in (qc, kc, vc))
        sq, sk, sv = (np.ascontiguousarray(a, dtype=np.float32) for a in (sq, sk, sv))
        BH, Lq, D = qc.shape
        Lk = kc.shape[1]
        if kc.shape != (BH, Lk, D) or vc.shape != (BH, Lk, D) or sq.shape != (BH, Lq) or sk.shape != (BH, Lk) \
                or sv.shape != (BH, Lk):
            raise ValueError("attention shapes disagree")
        out = np.empty((BH, Lq, D), np.float64)
        self.L.oracle_attention_i8(_p(qc), _p(sq), _p(kc), _p(sk), _p(vc), _p(sv), BH, Lq, Lk, D,
                                   float(1.0 / np.sqrt(D) if scale is None else scale), _p(out))
        return out

    def attention_probs(self, qc, sq, kc, sk, scale=None) -> np.ndarray:
        """Softmax probabilities of INT8 attention on codes: float64 [BH, Lq, Lk],
        each row summing to 1 (the reading in qdiff_oracle.c)."""
        qc, kc = (np.ascontiguousarray(a, dtype=np.int8) for a in (qc, kc))
        sq, sk = (np.ascontiguousarray(a, dtype=np.float32) for a in (sq, sk))
        BH, Lq, D = qc.shape
        Lk = kc.shape[1]
        if kc.shape != (BH, Lk, D) or sq.shape != (BH, Lq) or sk.shape != (BH, Lk):
            raise ValueError("attention shapes disagree")
        P = np.empty((BH, Lq, Lk), np.float64)
        self.L.oracle_attention_probs(_p(qc), _p(sq), _p(kc), _p(sk), BH, Lq, Lk, D,
                                      float(1.0 / np.sqrt(D) if scale is None else scale), _p(P))
        return P

    def quantize_tokens(self, x, dtype: str = "bf16"):
        """Per-token INT8 codes and scales of x [BH, L, D] (the unrotated row rule)."""
        x = np.asarray(x)
        BH, L, D = x.shape
        q, s = self.quantize_rowwise(x.reshape(BH * L, D), dtype, 0)
        return q.reshape(BH, L, D), s.reshape(BH, L)

    def attention(self, q, k, v, dtype: str = "bf16", scale=None) -> np.ndarray:
        """int8_attention of q [BH, Lq, D], k / v [BH, Lk, D] (16-bit bits or float32):
        per-token quantization of all three, then attention_codes."""
        qc, sq = self.quantize_tokens(q, dtype)
        kc, sk = self.quantize_tokens(k, dtype)
        vc, sv = self.quantize_tokens(v, dtype)
        return self.attention_codes(qc, sq, kc, sk, vc, sv, scale)

    def dequantize(self, q, scale, per_row: bool = True, out: str = "f32") -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        M, K = q.shape
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        res = np.empty((M, K), np.float32 if out == "f32" else np.uint16)
        self.L.oracle_dequantize(_p(q), M, K, K, _p(scale), int(per_row), int(out == "bf16"), _p(res))
        return res

    def pack_int4(self, q) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        R, K = q.shape
        if K % 2:
            raise ValueError("K must be even")
        out = np.empty((R, K // 2), np.uint8)
        self.L.oracle_pack_int4(_p(q), R, K, _p(out))
        return out

    def unpack_int4(self, packed, K: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        R = packed.shape[0]
        out = np.empty((R, K), np.int8)
        self.L.oracle_unpack_int4(_p(packed), R, K, _p(out))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def __getattr__(name):
    # module-level convenience: oracle.quantize_rowwise(...) etc.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
