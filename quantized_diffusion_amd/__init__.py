"""Rotated, dynamically quantized INT8 linear layer for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/qdiff.h`` (``libqdiff.so``,
built in-tree by ``python -m quantized_diffusion_amd.build``).  PyTorch only
supplies device memory and the current stream: every step of the layer runs
in the library's HIP kernels.  There is no fallback: if the library is
missing, or a tensor is not on the GPU, the call raises.

Operations (names as on the comfy-kitchen 0.2.40 page, "Huawei Ascend
backend"):
  quantize_and_rotate_rowwise(x)        -> (int8 codes, fp32 row scales)
  quantize_int8_rowwise(x)              -> (int8 codes, fp32 row scales)
  int8_linear(x, wq, w_scale, bias)     -> bf16 y = x W^T + b (rotated W8A8)
  dequantize_int8(q, scale, dtype)      -> fp32 / bf16
plus
  prepare_weights(W)                    -> offline (wq, w_scale) for int8_linear
  int8_scaled_mm(aq, a_scale, wq, w_scale, bias) -> bf16 (GEMM half of int8_linear)
  int8_gemm_i32(aq, wq)                 -> raw int32 accumulators
  quantize_and_rotate_rowwise_int4(x)   -> INT4 codes in int8 storage
  pack_int4(q), prepare_weights_w4a4(W) -> packed INT4 weights (two per byte)
  convrot_w4a4_linear(x, wp, w_scale, bias) -> bf16 y through the rotated INT4 path
  int4_scaled_mm / int4_gemm_i32        -> the packed-INT4 GEMM alone
  slice_weights(wq) -> K-sliced INT8 weights; int8_linear_sliced / int8_scaled_mm_sliced /
  int8_gemm_i32_sliced                  -> the same results with the faster weight layout
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LIB_PATH", "QDiffError", "lib", "quantize_and_rotate_rowwise", "quantize_and_rotate_rowwise_int4",
    "quantize_int8_rowwise", "int8_linear", "int8_scaled_mm", "int8_gemm_i32", "dequantize_int8",
    "prepare_weights", "workspace_size", "EXPORTED_SYMBOLS", "pack_int4", "prepare_weights_w4a4",
    "int4_scaled_mm", "int4_gemm_i32", "convrot_w4a4_linear", "quantize_int8_tensorwise",
    "tensorwise_workspace_size", "int8_scaled_mm_ex", "input_act", "quantize_rowwise_act", "int8_linear_act",
    "ACT_NONE", "ACT_GELU_TANH", "ACT_GELU_ERF", "ACT_SILU", "ACT_RELU", "pack_fp6", "fp6_scaled_mm",
    "fp6_gemm_i32", "w4a4_fp6_workspace_size", "convrot_w4a4_linear_fp6", "prepare_weights_w4a4_fp6",
    "quantize_and_rotate_rowwise_fp6", "set_gemm_tiles", "int8_gemm_tiles", "GEMM_TILES_AUTO", "GEMM_TILES_256x256",
    "GEMM_TILES_256x384", "int8_attention", "attention_workspace_size", "int8_attention_codes",
    "slice_weights", "int8_linear_sliced", "int8_scaled_mm_sliced", "int8_gemm_i32_sliced",
    "quantize_and_rotate_rowwise_sliced", "fp6_slice_weights", "quantize_and_rotate_rowwise_fp6_sliced",
    "fp6_scaled_mm_sliced", "fp6_gemm_i32_sliced", "convrot_w4a4_linear_fp6_sliced",
    "quantize_int8_tensorwise_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqdiff.so")

QD_OK, QD_EINVAL, QD_EUNSUPPORTED, QD_EHIP = 0, 1, 2, 3
QD_F32, QD_BF16, QD_F16 = 0, 1, 2
ACT_NONE, ACT_GELU_TANH, ACT_GELU_ERF, ACT_SILU, ACT_RELU = 0, 1, 2, 3, 4
GEMM_TILES_AUTO, GEMM_TILES_256x256, GEMM_TILES_256x384 = 0, 1, 2

EXPORTED_SYMBOLS = (
    "qd_last_error", "qd_version", "qd_quantize_and_rotate_rowwise",
    "qd_quantize_and_rotate_rowwise_int4", "qd_quantize_int8_rowwise", "qd_int8_scaled_mm",
    "qd_int8_linear_workspace_size", "qd_int8_linear", "qd_dequantize_int8", "qd_int8_gemm_i32",
    "qd_pack_int4", "qd_int4_scaled_mm", "qd_int4_gemm_i32", "qd_convrot_w4a4_linear",
    "qd_quantize_tensorwise_workspace_size", "qd_quantize_int8_tensorwise", "qd_int8_scaled_mm_ex",
    "qd_int8_linear_act", "qd_quantize_rowwise_act", "qd_input_act", "qd_pack_fp6", "qd_fp6_scaled_mm",
    "qd_fp6_gemm_i32", "qd_w4a4_fp6_workspace_size", "qd_convrot_w4a4_linear_fp6",
    "qd_quantize_and_rotate_rowwise_fp6", "qd_set_gemm_tiles", "qd_int8_gemm_tiles",
    "qd_int8_attention_workspace_size", "qd_int8_attention", "qd_int8_attention_codes",
    "qd_int8_slice_weights", "qd_int8_linear_sliced", "qd_int8_scaled_mm_sliced", "qd_int8_gemm_i32_sliced",
    "qd_quantize_and_rotate_rowwise_sliced", "qd_fp6_slice_weights", "qd_quantize_and_rotate_rowwise_fp6_sliced",
    "qd_fp6_scaled_mm_sliced", "qd_fp6_gemm_i32_sliced", "qd_convrot_w4a4_linear_fp6_sliced",
    "qd_quantize_int8_tensorwise_noalloc",
)


class QDiffError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libqdiff.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with "
                              "`python -m quantized_diffusion_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        St = ctypes.c_int
        L.qd_last_error.restype = ctypes.c_char_p
        L.qd_version.restype = ctypes.c_char_p
        L.qd_quantize_and_rotate_rowwise.restype = St
        L.qd_quantize_and_rotate_rowwise.argtypes = [P, St, I64, I64, I64, I32, P, I64, P, P]
        L.qd_quantize_and_rotate_rowwise_int4.restype = St
        L.qd_quantize_and_rotate_rowwise_int4.argtypes = [P, St, I64, I64, I64, I32, P, I64, P, P]
        L.qd_quantize_int8_rowwise.restype = St
        L.qd_quantize_int8_rowwise.argtypes = [P, St, I64, I64, I64, P, I64, P, P]
        L.qd_int8_scaled_mm.restype = St
        L.qd_int8_scaled_mm.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, P, I64, P]
        L.qd_int8_linear_workspace_size.restype = SZ
        L.qd_int8_linear_workspace_size.argtypes = [I64, I64]
        L.qd_int8_linear.restype = St
        L.qd_int8_linear.argtypes = [P, St, I64, I64, I64, P, I64, I64, P, P, I32, P, SZ, P, I64, P]
        L.qd_dequantize_int8.restype = St
        L.qd_dequantize_int8.argtypes = [P, I64, I64, I64, P, I32, St, P, I64, P]
        L.qd_int8_gemm_i32.restype = St
        L.qd_int8_attention_workspace_size.restype = SZ
        L.qd_int8_attention_workspace_size.argtypes = [I64, I64, I64, I64]
        L.qd_int8_attention.restype = St
        L.qd_int8_attention.argtypes = [P, P, P, St, I64, I64, I64, I64, ctypes.c_float, P, SZ, P, P]
        L.qd_int8_attention_codes.restype = St
        L.qd_int8_attention_codes.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_float, P, P]
        L.qd_set_gemm_tiles.restype = St
        L.qd_set_gemm_tiles.argtypes = [St]
        L.qd_int8_gemm_tiles.restype = St
        L.qd_int8_gemm_tiles.argtypes = [I64, I64, I64]
        L.qd_int8_gemm_i32.argtypes = [P, I64, I64, I64, P, I64, I64, P, I64, P]
        L.qd_pack_int4.restype = St
        L.qd_pack_int4.argtypes = [P, I64, I64, I64, P, I64, P]
        L.qd_int4_scaled_mm.restype = St
        L.qd_int4_scaled_mm.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, P, I64, P]
        L.qd_int4_gemm_i32.restype = St
        L.qd_int4_gemm_i32.argtypes = [P, I64, I64, I64, P, I64, I64, P, I64, P]
        L.qd_convrot_w4a4_linear.restype = St
        L.qd_convrot_w4a4_linear.argtypes = [P, St, I64, I64, I64, P, I64, I64, P, P, I32, P, SZ, P, I64, P]
        L.qd_quantize_tensorwise_workspace_size.restype = SZ
        L.qd_quantize_tensorwise_workspace_size.argtypes = []
        L.qd_quantize_int8_tensorwise.restype = St
        L.qd_quantize_int8_tensorwise.argtypes = [P, St, I64, I64, I64, P, I64, P, P, SZ, P]
        L.qd_quantize_int8_tensorwise_noalloc.restype = St
        L.qd_quantize_int8_tensorwise_noalloc.argtypes = [P, St, I64, I64, I64, P, I64, P, P]
        L.qd_int8_scaled_mm_ex.restype = St
        L.qd_int8_scaled_mm_ex.argtypes = [P, I64, I64, I64, P, I64, P, I64, I64, P, I64, P, P, I64, P]
        L.qd_int8_linear_act.restype = St
        L.qd_int8_linear_act.argtypes = [P, St, I64, I64, I64, St, P, I64, I64, P, P, I32, P, SZ, P, I64, P]
        L.qd_quantize_rowwise_act.restype = St
        L.qd_quantize_rowwise_act.argtypes = [P, St, I64, I64, I64, St, I32, P, I64, P, P]
        L.qd_input_act.restype = St
        L.qd_input_act.argtypes = [P, St, I64, St, P, P]
        L.qd_pack_fp6.restype = St
        L.qd_pack_fp6.argtypes = [P, I64, I64, I64, P, I64, P]
        L.qd_fp6_scaled_mm.restype = St
        L.qd_fp6_scaled_mm.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, P, I64, P]
        L.qd_fp6_gemm_i32.restype = St
        L.qd_fp6_gemm_i32.argtypes = [P, I64, I64, I64, P, I64, I64, P, I64, P]
        L.qd_w4a4_fp6_workspace_size.restype = SZ
        L.qd_w4a4_fp6_workspace_size.argtypes = [I64, I64]
        L.qd_quantize_and_rotate_rowwise_fp6.restype = St
        L.qd_quantize_and_rotate_rowwise_fp6.argtypes = [P, St, I64, I64, I64, I32, P, I64, P, P]
        L.qd_convrot_w4a4_linear_fp6.restype = St
        L.qd_convrot_w4a4_linear_fp6.argtypes = [P, St, I64, I64, I64, P, I64, I64, P, P, I32, P, SZ, P, I64, P]
        L.qd_int8_slice_weights.restype = St
        L.qd_int8_slice_weights.argtypes = [P, I64, I64, I64, P, P]
        L.qd_int8_linear_sliced.restype = St
        L.qd_int8_linear_sliced.argtypes = [P, St, I64, I64, I64, St, P, I64, P, P, I32, P, SZ, P, I64, P]
        L.qd_int8_scaled_mm_sliced.restype = St
        L.qd_int8_scaled_mm_sliced.argtypes = [P, I64, I64, I64, I32, P, P, I64, P, P, P, I64, P]
        L.qd_quantize_and_rotate_rowwise_sliced.restype = St
        L.qd_quantize_and_rotate_rowwise_sliced.argtypes = [P, St, I64, I64, I64, St, I32, P, P, P]
        L.qd_int8_gemm_i32_sliced.restype = St
        L.qd_int8_gemm_i32_sliced.argtypes = [P, I64, I64, I64, I32, P, I64, P, I64, P]
        L.qd_fp6_slice_weights.restype = St
        L.qd_fp6_slice_weights.argtypes = [P, I64, I64, I64, P, P]
        L.qd_quantize_and_rotate_rowwise_fp6_sliced.restype = St
        L.qd_quantize_and_rotate_rowwise_fp6_sliced.argtypes = [P, St, I64, I64, I64, I32, P, P, P]
        L.qd_fp6_scaled_mm_sliced.restype = St
        L.qd_fp6_scaled_mm_sliced.argtypes = [P, I64, I64, I64, I32, P, P, I64, P, P, P, I64, P]
        L.qd_fp6_gemm_i32_sliced.restype = St
        L.qd_fp6_gemm_i32_sliced.argtypes = [P, I64, I64, I64, I32, P, I64, P, I64, P]
        L.qd_convrot_w4a4_linear_fp6_sliced.restype = St
        L.qd_convrot_w4a4_linear_fp6_sliced.argtypes = [P, St, I64, I64, I64, P, I64, P, P, I32, P, SZ, P, I64, P]
        _lib = L
    return _lib


def _check(status: int):
    if status != QD_OK:
        raise QDiffError(status, lib().qd_last_error().decode())


# --------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: QD_F32, torch.bfloat16: QD_BF16, torch.float16: QD_F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("qdiff: tensors must be on the GPU (no CPU fallback)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("qdiff: tensors are on different devices")
    return dev


def _mat(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return t


def _out(t, shape, dtype, name="out"):
    """A caller-provided output: dtype and shape exactly as the call writes
    them, rows with a contiguous last dimension (2-D) or fully contiguous
    (other ranks), so that no kernel writes past the tensor."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.dim() == 2:
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
        if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
            raise ValueError(f"{name} rows overlap (row stride {t.stride(0)} < {t.shape[1]})")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bf16_out(M, N, dev):
    """BF16 [M, N] output whose row stride is a multiple of 8 elements (the
    GEMM stores 16 bytes at a time)."""
    torch = _torch()
    return torch.empty((M, (N + 7) // 8 * 8), dtype=torch.bfloat16, device=dev)[:, :N]


def _rows_vec(t, n, dtype, name):
    torch = _torch()
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] < n or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D {dtype} tensor of length >= {n}")
    return t


# ------------------------------------------------------------------ quantizers

def _quantize(fn, x, block, out_q, out_scale, rotate: bool):
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q, out_scale)
    M, K = x.shape
    ldq = (K + 15) // 16 * 16
    if out_q is None:
        buf = torch.empty((M, ldq), dtype=torch.int8, device=dev)
        out_q = buf[:, :K]
    if out_scale is None:
        out_scale = torch.empty(M, dtype=torch.float32, device=dev)
    _out(out_q, (M, K), torch.int8, "out_q")
    _out(out_scale, (M,), torch.float32, "out_scale")
    args = [_ptr(x), _dtype_code(x), M, K, x.stride(0)]
    if rotate:
        args.append(block)
    args += [_ptr(out_q), out_q.stride(0), _ptr(out_scale), _stream(dev)]
    _check(fn(*args))
    return out_q, out_scale


def quantize_and_rotate_rowwise(x, block: int = 256, out_q=None, out_scale=None):
    """Rotate each 256-block of the rows of x (FP32/BF16/FP16 [M, K]) by the
    normalised Walsh-Hadamard transform, then quantize each row to INT8.
    Returns (codes int8 [M, K], row scales fp32 [M])."""
    return _quantize(lib().qd_quantize_and_rotate_rowwise, x, block, out_q, out_scale, True)


def quantize_and_rotate_rowwise_int4(x, block: int = 256, out_q=None, out_scale=None):
    """As quantize_and_rotate_rowwise with INT4 codes in [-7, 7] (int8 storage), s = amax/7."""
    return _quantize(lib().qd_quantize_and_rotate_rowwise_int4, x, block, out_q, out_scale, True)


def quantize_int8_rowwise(x, out_q=None, out_scale=None):
    """Per-row dynamic symmetric INT8 quantization (no rotation)."""
    return _quantize(lib().qd_quantize_int8_rowwise, x, 0, out_q, out_scale, False)


def tensorwise_workspace_size() -> int:
    """Bytes of workspace quantize_int8_tensorwise needs (partial maxima)."""
    return int(lib().qd_quantize_tensorwise_workspace_size())


def quantize_int8_tensorwise(x, out_q=None, out_scale=None, workspace=None):
    """Tensor-wise dynamic symmetric INT8 quantization (no rotation): one FP32
    scale s = max|x| / 127 for the whole tensor.  Returns (codes int8 [M, K],
    scale fp32 [1])."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q, out_scale, workspace)
    M, K = x.shape
    if out_q is None:
        out_q = torch.empty((M, (K + 15) // 16 * 16), dtype=torch.int8, device=dev)[:, :K]
    if out_scale is None:
        out_scale = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(tensorwise_workspace_size(), dtype=torch.uint8, device=dev)
    _out(out_q, (M, K), torch.int8, "out_q")
    _out(out_scale, (1,), torch.float32, "out_scale")
    _check(lib().qd_quantize_int8_tensorwise(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(out_q),
                                             out_q.stride(0), _ptr(out_scale), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(dev)))
    return out_q, out_scale


def quantize_int8_tensorwise_noalloc(x, out_q, out_scale):
    """quantize_int8_tensorwise through the library's allocation-free entry
    point: the caller passes the outputs (codes int8 [M, K], scale fp32 [1]);
    the partial maxima live in the library's fixed per-GPU array, so nothing
    is allocated.  Calls overlapping on one GPU race (see qdiff.h)."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q, out_scale)
    M, K = x.shape
    _out(out_q, (M, K), torch.int8, "out_q")
    _out(out_scale, (1,), torch.float32, "out_scale")
    _check(lib().qd_quantize_int8_tensorwise_noalloc(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(out_q),
                                                     out_q.stride(0), _ptr(out_scale), _stream(dev)))
    return out_q, out_scale


def prepare_weights(w, block: int = 256):
    """Offline weight preparation for int8_linear: rotate FP32 W [N, K] along K
    (block 256, or 0 for none) and quantize per output channel.
    Returns (wq int8 [N, K], w_scale fp32 [N])."""
    if block == 0:
        return quantize_int8_rowwise(w)
    return quantize_and_rotate_rowwise(w, block)


# ------------------------------------------------------------------------ GEMMs

def int8_scaled_mm(aq, a_scale, wq, w_scale, bias=None, out=None):
    """y[m, n] = bf16(((float)(aq . wq^T)[m, n] * a_scale[m]) * w_scale[n] + bias[n])."""
    torch = _torch()
    _mat(aq, "aq"), _mat(wq, "wq")
    dev = _dev(aq, a_scale, wq, w_scale, bias, out)
    M, K = aq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("aq and wq disagree on K")
    _rows_vec(a_scale, M, torch.float32, "a_scale")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_scaled_mm(_ptr(aq), M, K, aq.stride(0), _ptr(a_scale), _ptr(wq), N, wq.stride(0),
                                   _ptr(w_scale), _ptr(bias), _ptr(out), out.stride(0), _stream(dev)))
    return out


def int8_scaled_mm_ex(aq, a_scale, wq, w_scale, bias=None, out=None):
    """int8_scaled_mm with per-tensor scales allowed: a_scale of length M (per
    row) or 1 (one for all rows), w_scale of length N (per output channel) or 1."""
    torch = _torch()
    _mat(aq, "aq"), _mat(wq, "wq")
    dev = _dev(aq, a_scale, wq, w_scale, bias, out)
    M, K = aq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("aq and wq disagree on K")
    for t, name in ((a_scale, "a_scale"), (w_scale, "w_scale")):
        if t.dtype != torch.float32 or t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous 1-D float32 tensor")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_scaled_mm_ex(_ptr(aq), M, K, aq.stride(0), _ptr(a_scale), a_scale.numel(), _ptr(wq), N,
                                      wq.stride(0), _ptr(w_scale), w_scale.numel(), _ptr(bias), _ptr(out),
                                      out.stride(0), _stream(dev)))
    return out


def int8_gemm_i32(aq, wq, out=None):
    """Raw int32 accumulators aq . wq^T of the same GEMM kernel."""
    torch = _torch()
    _mat(aq, "aq"), _mat(wq, "wq")
    dev = _dev(aq, wq, out)
    M, K = aq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("aq and wq disagree on K")
    if out is None:
        ldc = (N + 3) // 4 * 4
        out = torch.empty((M, ldc), dtype=torch.int32, device=dev)[:, :N]
    _out(out, (M, N), torch.int32)
    _check(lib().qd_int8_gemm_i32(_ptr(aq), M, K, aq.stride(0), _ptr(wq), N, wq.stride(0), _ptr(out),
                                  out.stride(0), _stream(dev)))
    return out


# --------------------------------------------------- K-sliced INT8 weights

def _sliced(w, name="w_sliced"):
    """(K, N) of K-sliced weights: a contiguous int8 tensor [K / 64, N, 64]."""
    torch = _torch()
    if w.dtype != torch.int8 or w.dim() != 3 or w.shape[2] != 64 or not w.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int8 tensor [K / 64, N, 64] (from slice_weights)")
    return w.shape[0] * 64, w.shape[1]


def slice_weights(wq, out=None):
    """Row-major INT8 weight codes wq [N, K] (K % 64 == 0) -> the K-sliced
    layout the GEMM reads faster: int8 [K / 64, N, 64], element [u, n, j] =
    wq[n, 64 u + j].  Offline, like prepare_weights."""
    torch = _torch()
    _mat(wq, "wq")
    dev = _dev(wq, out)
    N, K = wq.shape
    if out is None:
        out = torch.empty((max(K // 64, 0), N, 64), dtype=torch.int8, device=dev)
    _out(out, (K // 64, N, 64), torch.int8)
    _check(lib().qd_int8_slice_weights(_ptr(wq), N, K, wq.stride(0), _ptr(out), _stream(dev)))
    return out


def int8_linear_sliced(x, w_sliced, w_scale, bias=None, input_act: int = ACT_NONE, rotate_block: int = 256,
                       workspace=None, out=None):
    """int8_linear_act with K-sliced weights (slice_weights of prepare_weights'
    codes): identical results, faster GEMM."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, w_sliced, w_scale, bias, workspace, out)
    M, K = x.shape
    Kw, N = _sliced(w_sliced)
    if Kw != K:
        raise ValueError("x and w_sliced disagree on K")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if workspace is None:
        workspace = torch.empty(max(workspace_size(M, K), 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_linear_sliced(_ptr(x), _dtype_code(x), M, K, x.stride(0), int(input_act), _ptr(w_sliced),
                                       N, _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0),
                                       _stream(dev)))
    return out


def _a_operand(aq, name="aq"):
    """(M, K, lda, a_sliced) of activation codes: row-major int8 [M, K] or K-sliced [K / 64, M, 64]."""
    if aq.dim() == 3:
        K, M = _sliced(aq, name)
        return M, K, K, 1
    _mat(aq, name)
    return aq.shape[0], aq.shape[1], aq.stride(0), 0


def quantize_and_rotate_rowwise_sliced(x, block: int = 256, out_q=None, out_scale=None, input_act: int = ACT_NONE):
    """quantize_and_rotate_rowwise (with input_act: quantize_rowwise_act) with the
    codes in the K-sliced layout: returns (int8 [K / 64, M, 64], fp32 row scales [M])."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q, out_scale)
    M, K = x.shape
    if out_q is None:
        out_q = torch.empty((max(K // 64, 0), M, 64), dtype=torch.int8, device=dev)
    if out_scale is None:
        out_scale = torch.empty(M, dtype=torch.float32, device=dev)
    _out(out_q, (K // 64, M, 64), torch.int8, "out_q")
    _out(out_scale, (M,), torch.float32, "out_scale")
    _check(lib().qd_quantize_and_rotate_rowwise_sliced(_ptr(x), _dtype_code(x), M, K, x.stride(0), int(input_act),
                                                       block, _ptr(out_q), _ptr(out_scale), _stream(dev)))
    return out_q, out_scale


def int8_scaled_mm_sliced(aq, a_scale, w_sliced, w_scale, bias=None, out=None):
    """int8_scaled_mm with K-sliced weights; aq row-major [M, K] or K-sliced
    [K / 64, M, 64].  Identical results."""
    torch = _torch()
    dev = _dev(aq, a_scale, w_sliced, w_scale, bias, out)
    M, K, lda, a_sl = _a_operand(aq)
    Kw, N = _sliced(w_sliced)
    if Kw != K:
        raise ValueError("aq and w_sliced disagree on K")
    _rows_vec(a_scale, M, torch.float32, "a_scale")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_scaled_mm_sliced(_ptr(aq), M, K, lda, a_sl, _ptr(a_scale), _ptr(w_sliced), N,
                                          _ptr(w_scale), _ptr(bias), _ptr(out), out.stride(0), _stream(dev)))
    return out


def int8_gemm_i32_sliced(aq, w_sliced, out=None):
    """int8_gemm_i32 with K-sliced weights (aq as in int8_scaled_mm_sliced): identical accumulators."""
    torch = _torch()
    dev = _dev(aq, w_sliced, out)
    M, K, lda, a_sl = _a_operand(aq)
    Kw, N = _sliced(w_sliced)
    if Kw != K:
        raise ValueError("aq and w_sliced disagree on K")
    if out is None:
        out = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.int32, device=dev)[:, :N]
    _out(out, (M, N), torch.int32)
    _check(lib().qd_int8_gemm_i32_sliced(_ptr(aq), M, K, lda, a_sl, _ptr(w_sliced), N, _ptr(out),
                                         out.stride(0), _stream(dev)))
    return out


def attention_workspace_size(BH: int, Lq: int, Lk: int, D: int) -> int:
    return int(lib().qd_int8_attention_workspace_size(BH, Lq, Lk, D))


def int8_attention(q, k, v, scale: float = 0.0, workspace=None, out=None):
    """INT8 attention of q [BH, Lq, D], k / v [BH, Lk, D] (contiguous, same
    dtype: float32, bfloat16 or float16; D = 64 or 128) -> BF16 [BH, Lq, D].
    scale <= 0: 1/sqrt(D).  The workspace (optional) ends up holding the
    per-token codes and scales (qdiff.h gives the layout)."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [BH, L, D]")
    BH, Lq, D = q.shape
    Lk = k.shape[1]
    if k.shape != (BH, Lk, D) or v.shape != (BH, Lk, D):
        raise ValueError("q, k, v shapes disagree")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dev = _dev(q, k, v, out)
    if workspace is None:
        workspace = torch.empty(max(1, attention_workspace_size(BH, Lq, Lk, D)), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((BH, Lq, D), dtype=torch.bfloat16, device=dev)
    _out(out, (BH, Lq, D), torch.bfloat16)
    _check(lib().qd_int8_attention(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), BH, Lq, Lk, D, float(scale),
                                   _ptr(workspace), workspace.numel(), _ptr(out), _stream(dev)))
    return out


def int8_attention_codes(qc, sq, kc, sk, vc, sv, scale: float = 0.0, out=None):
    """The attention step on per-token codes: qc [BH, Lq, D] / kc, vc [BH, Lk, D]
    int8 and scales sq [BH, Lq] / sk, sv [BH, Lk] float32 -> BF16 [BH, Lq, D]."""
    torch = _torch()
    BH, Lq, D = qc.shape
    Lk = kc.shape[1]
    if kc.shape != (BH, Lk, D) or vc.shape != (BH, Lk, D) or sq.shape != (BH, Lq) or sk.shape != (BH, Lk) \
            or sv.shape != (BH, Lk):
        raise ValueError("code / scale shapes disagree")
    for t, n in ((qc, "qc"), (kc, "kc"), (vc, "vc"), (sq, "sq"), (sk, "sk"), (sv, "sv")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dev = _dev(qc, sq, kc, sk, vc, sv, out)
    if out is None:
        out = torch.empty((BH, Lq, D), dtype=torch.bfloat16, device=dev)
    _out(out, (BH, Lq, D), torch.bfloat16)
    _check(lib().qd_int8_attention_codes(_ptr(qc), _ptr(sq), _ptr(kc), _ptr(sk), _ptr(vc), _ptr(sv), BH, Lq, Lk,
                                         D, float(scale), _ptr(out), _stream(dev)))
    return out


def set_gemm_tiles(tiles: int) -> None:
    """Output tile of the INT8-weight GEMM kernels for every later launch in
    the process: GEMM_TILES_AUTO (chosen by shape, the default),
    GEMM_TILES_256x256 or GEMM_TILES_256x384.  Results are identical."""
    _check(lib().qd_set_gemm_tiles(int(tiles)))


def int8_gemm_tiles(M: int, N: int, K: int) -> int:
    """GEMM_TILES_256x256 or GEMM_TILES_256x384: the tile an INT8-weight GEMM
    of this shape uses under the current setting."""
    return int(lib().qd_int8_gemm_tiles(M, N, K))


def workspace_size(M: int, K: int) -> int:
    return int(lib().qd_int8_linear_workspace_size(M, K))


def int8_linear(x, wq, w_scale, bias=None, rotate_block: int = 256, workspace=None, out=None):
    """y = x W^T + b through the rotated INT8 path (two kernels: rotate+quantize,
    then INT8 GEMM with the fused dequantizing epilogue).  wq/w_scale must come
    from prepare_weights with the same rotate_block.  Returns bf16 [M, N]."""
    torch = _torch()
    _mat(x, "x"), _mat(wq, "wq")
    dev = _dev(x, wq, w_scale, bias, workspace, out)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("x and wq disagree on K")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    need = workspace_size(M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_linear(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(wq), N, wq.stride(0),
                                _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0),
                                _stream(dev)))
    return out


def int8_linear_act(x, wq, w_scale, bias=None, input_act: int = ACT_NONE, rotate_block: int = 256,
                    workspace=None, out=None):
    """int8_linear(input_act=...): y = act(x) W^T + b, the activation applied in
    the quantizer's load (act(x) rounded to x's dtype, BF16 or FP16)."""
    torch = _torch()
    _mat(x, "x"), _mat(wq, "wq")
    dev = _dev(x, wq, w_scale, bias, workspace, out)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("x and wq disagree on K")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    need = workspace_size(M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int8_linear_act(_ptr(x), _dtype_code(x), M, K, x.stride(0), int(input_act), _ptr(wq), N,
                                    wq.stride(0), _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0),
                                    _stream(dev)))
    return out


def quantize_rowwise_act(x, input_act: int, rotate_block: int = 256, out_q=None, out_scale=None):
    """Codes and row scales of act(x) (rotated when rotate_block == 256)."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q, out_scale)
    M, K = x.shape
    if out_q is None:
        out_q = torch.empty((M, (K + 15) // 16 * 16), dtype=torch.int8, device=dev)[:, :K]
    if out_scale is None:
        out_scale = torch.empty(M, dtype=torch.float32, device=dev)
    _out(out_q, (M, K), torch.int8, "out_q")
    _out(out_scale, (M,), torch.float32, "out_scale")
    _check(lib().qd_quantize_rowwise_act(_ptr(x), _dtype_code(x), M, K, x.stride(0), int(input_act), rotate_block,
                                         _ptr(out_q), out_q.stride(0), _ptr(out_scale), _stream(dev)))
    return out_q, out_scale


def input_act(x, act: int, out=None):
    """act(x) elementwise in x's 16-bit dtype (the quantizer's activation, alone)."""
    torch = _torch()
    dev = _dev(x, out)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    _out(out, tuple(x.shape), x.dtype)
    _check(lib().qd_input_act(_ptr(x), _dtype_code(x), x.numel(), int(act), _ptr(out), _stream(dev)))
    return out


# ------------------------------------------------------------- FP6 operands

def _f6_ld(K):
    return (K // 4 * 3 + 15) // 16 * 16


def pack_fp6(q, out=None):
    """INT4 codes (int8 [R, K], values in [-7, 7]) -> the FP6 E2M3 operand format
    (uint8 [R, 3K/4]), exact for every code."""
    torch = _torch()
    _mat(q, "q")
    dev = _dev(q, out)
    R, K = q.shape
    if out is None:
        out = torch.empty((R, _f6_ld(K)), dtype=torch.uint8, device=dev)[:, :K // 4 * 3]
    _out(out, (R, K // 4 * 3), torch.uint8)
    _check(lib().qd_pack_fp6(_ptr(q), R, K, q.stride(0), _ptr(out), out.stride(0), _stream(dev)))
    return out


def quantize_and_rotate_rowwise_fp6(x, block: int = 256, out_q6=None, out_scale=None):
    """Rotating INT4 quantizer writing the FP6 operand format (BF16/FP16 x):
    returns (q6 uint8 [M, 3K/4], row scales fp32 [M])."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q6, out_scale)
    M, K = x.shape
    if out_q6 is None:
        out_q6 = torch.empty((M, _f6_ld(K)), dtype=torch.uint8, device=dev)[:, :K // 4 * 3]
    if out_scale is None:
        out_scale = torch.empty(M, dtype=torch.float32, device=dev)
    _out(out_q6, (M, K // 4 * 3), torch.uint8, "out_q6")
    _out(out_scale, (M,), torch.float32, "out_scale")
    _check(lib().qd_quantize_and_rotate_rowwise_fp6(_ptr(x), _dtype_code(x), M, K, x.stride(0), block,
                                                    _ptr(out_q6), out_q6.stride(0), _ptr(out_scale), _stream(dev)))
    return out_q6, out_scale


def prepare_weights_w4a4_fp6(w, block: int = 256):
    """Offline W4A4 weights for the FP6 path: rotate, quantize per channel to INT4
    codes, pack as FP6.  Returns (w6 uint8 [N, 3K/4], w_scale fp32 [N])."""
    q, s = quantize_and_rotate_rowwise_int4(w, block)
    return pack_fp6(q), s


def _f6_rows(t, K, name):
    _mat(t, name)
    if t.shape[1] != K // 4 * 3:
        raise ValueError(f"{name} must hold 3K/4 = {K // 4 * 3} bytes per row, got {t.shape[1]}")
    return t


def fp6_scaled_mm(a6, a_scale, w6, w_scale, K: int, bias=None, out=None):
    """The GEMM on FP6 operands (K values per row), BF16 out with the fused epilogue."""
    torch = _torch()
    _f6_rows(a6, K, "a6"), _f6_rows(w6, K, "w6")
    dev = _dev(a6, a_scale, w6, w_scale, bias, out)
    M, N = a6.shape[0], w6.shape[0]
    _rows_vec(a_scale, M, torch.float32, "a_scale")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_fp6_scaled_mm(_ptr(a6), M, K, a6.stride(0), _ptr(a_scale), _ptr(w6), N, w6.stride(0),
                                  _ptr(w_scale), _ptr(bias), _ptr(out), out.stride(0), _stream(dev)))
    return out


def fp6_gemm_i32(a6, w6, K: int, out=None):
    """Exact sums of the FP6 GEMM as int32 [M, N]."""
    torch = _torch()
    _f6_rows(a6, K, "a6"), _f6_rows(w6, K, "w6")
    dev = _dev(a6, w6, out)
    M, N = a6.shape[0], w6.shape[0]
    if out is None:
        out = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.int32, device=dev)[:, :N]
    _out(out, (M, N), torch.int32)
    _check(lib().qd_fp6_gemm_i32(_ptr(a6), M, K, a6.stride(0), _ptr(w6), N, w6.stride(0), _ptr(out),
                                 out.stride(0), _stream(dev)))
    return out


def w4a4_fp6_workspace_size(M: int, K: int) -> int:
    return int(lib().qd_w4a4_fp6_workspace_size(M, K))


def convrot_w4a4_linear_fp6(x, w6, w_scale, bias=None, rotate_block: int = 256, workspace=None, out=None):
    """convrot_w4a4_linear with FP6 weights (prepare_weights_w4a4_fp6): same results, FP6 matrix path."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, w6, w_scale, bias, workspace, out)
    M, K = x.shape
    _f6_rows(w6, K, "w6")
    N = w6.shape[0]
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if workspace is None:
        workspace = torch.empty(max(w4a4_fp6_workspace_size(M, K), 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_convrot_w4a4_linear_fp6(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(w6), N, w6.stride(0),
                                            _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0),
                                            _stream(dev)))
    return out


def _f6_sliced(w, name="w6_sliced"):
    """(K, R) of a K-sliced FP6 operand: a contiguous uint8 tensor [K / 128, R, 96]."""
    torch = _torch()
    if w.dtype != torch.uint8 or w.dim() != 3 or w.shape[2] != 96 or not w.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor [K / 128, R, 96] (K-sliced FP6)")
    return w.shape[0] * 128, w.shape[1]


def fp6_slice_weights(w6, K: int, out=None):
    """Row-major FP6 weights w6 [N, 3K/4] (K % 128 == 0) -> the K-sliced layout
    uint8 [K / 128, N, 96], element [u, n, j] = w6[n, 96 u + j].  Offline."""
    torch = _torch()
    _mat(w6, "w6")
    dev = _dev(w6, out)
    N = w6.shape[0]
    if out is None:
        out = torch.empty((max(K // 128, 0), N, 96), dtype=torch.uint8, device=dev)
    _out(out, (K // 128, N, 96), torch.uint8)
    if w6.shape[1] != K // 4 * 3:
        raise ValueError("w6 must hold 3K/4 bytes per row")
    _check(lib().qd_fp6_slice_weights(_ptr(w6), N, K, w6.stride(0), _ptr(out), _stream(dev)))
    return out


def quantize_and_rotate_rowwise_fp6_sliced(x, block: int = 256, out_q6=None, out_scale=None):
    """quantize_and_rotate_rowwise_fp6 with the K-sliced FP6 output: (uint8 [K / 128, M, 96], fp32 [M])."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, out_q6, out_scale)
    M, K = x.shape
    if out_q6 is None:
        out_q6 = torch.empty((max(K // 128, 0), M, 96), dtype=torch.uint8, device=dev)
    if out_scale is None:
        out_scale = torch.empty(M, dtype=torch.float32, device=dev)
    _out(out_q6, (K // 128, M, 96), torch.uint8, "out_q6")
    _out(out_scale, (M,), torch.float32, "out_scale")
    _check(lib().qd_quantize_and_rotate_rowwise_fp6_sliced(_ptr(x), _dtype_code(x), M, K, x.stride(0), block,
                                                           _ptr(out_q6), _ptr(out_scale), _stream(dev)))
    return out_q6, out_scale


def _f6_a_operand(a6, K):
    """(M, lda, a_sliced) of an FP6 activation operand: row-major [M, 3K/4] or K-sliced [K / 128, M, 96]."""
    if a6.dim() == 3:
        Ka, M = _f6_sliced(a6, "a6")
        if Ka != K:
            raise ValueError("a6 and w6_sliced disagree on K")
        return M, K // 4 * 3, 1
    _f6_rows(a6, K, "a6")
    return a6.shape[0], a6.stride(0), 0


def fp6_scaled_mm_sliced(a6, a_scale, w6_sliced, w_scale, bias=None, out=None):
    """fp6_scaled_mm with K-sliced FP6 weights (a6 row-major or K-sliced): identical results."""
    torch = _torch()
    dev = _dev(a6, a_scale, w6_sliced, w_scale, bias, out)
    K, N = _f6_sliced(w6_sliced)
    M, lda, a_sl = _f6_a_operand(a6, K)
    _rows_vec(a_scale, M, torch.float32, "a_scale")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_fp6_scaled_mm_sliced(_ptr(a6), M, K, lda, a_sl, _ptr(a_scale), _ptr(w6_sliced), N, _ptr(w_scale),
                                         _ptr(bias), _ptr(out), out.stride(0), _stream(dev)))
    return out


def fp6_gemm_i32_sliced(a6, w6_sliced, out=None):
    """fp6_gemm_i32 with K-sliced FP6 weights: identical exact sums."""
    torch = _torch()
    dev = _dev(a6, w6_sliced, out)
    K, N = _f6_sliced(w6_sliced)
    M, lda, a_sl = _f6_a_operand(a6, K)
    if out is None:
        out = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.int32, device=dev)[:, :N]
    _out(out, (M, N), torch.int32)
    _check(lib().qd_fp6_gemm_i32_sliced(_ptr(a6), M, K, lda, a_sl, _ptr(w6_sliced), N, _ptr(out), out.stride(0),
                                        _stream(dev)))
    return out


def convrot_w4a4_linear_fp6_sliced(x, w6_sliced, w_scale, bias=None, rotate_block: int = 256, workspace=None,
                                   out=None):
    """convrot_w4a4_linear_fp6 with K-sliced FP6 weights (fp6_slice_weights): identical results."""
    torch = _torch()
    _mat(x, "x")
    dev = _dev(x, w6_sliced, w_scale, bias, workspace, out)
    M, K = x.shape
    Kw, N = _f6_sliced(w6_sliced)
    if Kw != K:
        raise ValueError("x and w6_sliced disagree on K")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if workspace is None:
        workspace = torch.empty(max(w4a4_fp6_workspace_size(M, K), 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_convrot_w4a4_linear_fp6_sliced(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(w6_sliced), N,
                                                   _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                                   workspace.numel() * workspace.element_size(), _ptr(out),
                                                   out.stride(0), _stream(dev)))
    return out


# -------------------------------------------------------------- dequantization

def dequantize_int8(q, scale, out_dtype=None, out=None):
    """out = fl(q * s): s = scale[m] if scale has M entries, else scale[0] (per tensor)."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    _mat(q, "q")
    dev = _dev(q, scale, out)
    M, K = q.shape
    per_row = scale.numel() == M and M != 1
    if scale.dtype != torch.float32 or scale.numel() < 1 or (scale.numel() > 1 and scale.stride(0) != 1):
        raise ValueError("scale must be a non-empty contiguous fp32 tensor")
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=dev)
    _out(out, (M, K), out.dtype if out.dtype in (torch.float32, torch.bfloat16) else out_dtype)
    _check(lib().qd_dequantize_int8(_ptr(q), M, K, q.stride(0), _ptr(scale), int(per_row),
                                    _dtype_code(out), _ptr(out), out.stride(0), _stream(dev)))
    return out


# ------------------------------------------------------------ W4A4 (INT4) path

def pack_int4(q, out=None):
    """Pack INT4 codes (int8 storage, values in [-8, 7]) two per byte along K:
    byte i = (q[2i] & 15) | (q[2i+1] & 15) << 4.  Returns uint8 [R, K/2]."""
    torch = _torch()
    _mat(q, "q")
    dev = _dev(q, out)
    R, K = q.shape
    if out is None:
        ldp = (K // 2 + 15) // 16 * 16
        out = torch.empty((R, ldp), dtype=torch.uint8, device=dev)[:, : K // 2]
    _out(out, (R, K // 2), torch.uint8, "out")
    _check(lib().qd_pack_int4(_ptr(q), R, K, q.stride(0), _ptr(out), out.stride(0), _stream(dev)))
    return out


def prepare_weights_w4a4(w, block: int = 256):
    """Offline weight preparation for convrot_w4a4_linear: rotate FP32 W [N, K]
    along K, quantize per output channel to INT4 (s = amax/7), pack two codes
    per byte.  Returns (packed uint8 [N, K/2], w_scale fp32 [N])."""
    q, s = quantize_and_rotate_rowwise_int4(w, block)
    return pack_int4(q), s


def _w4_common(aq, wp, name):
    _mat(aq, "aq"), _mat(wp, name)
    M, K = aq.shape
    N = wp.shape[0]
    if wp.shape[1] * 2 != K:
        raise ValueError(f"{name} must be [N, K/2] packed bytes for K={K}")
    return M, K, N


def int4_scaled_mm(aq, a_scale, wp, w_scale, bias=None, out=None):
    """y = bf16(((float)(aq . unpack(wp)^T) * a_scale[m]) * w_scale[n] + bias[n])."""
    torch = _torch()
    M, K, N = _w4_common(aq, wp, "wp")
    dev = _dev(aq, a_scale, wp, w_scale, bias, out)
    _rows_vec(a_scale, M, torch.float32, "a_scale")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_int4_scaled_mm(_ptr(aq), M, K, aq.stride(0), _ptr(a_scale), _ptr(wp), N, wp.stride(0),
                                   _ptr(w_scale), _ptr(bias), _ptr(out), out.stride(0), _stream(dev)))
    return out


def int4_gemm_i32(aq, wp, out=None):
    """Raw int32 accumulators aq . unpack(wp)^T of the packed-INT4 GEMM kernel."""
    torch = _torch()
    M, K, N = _w4_common(aq, wp, "wp")
    dev = _dev(aq, wp, out)
    if out is None:
        out = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.int32, device=dev)[:, :N]
    _out(out, (M, N), torch.int32)
    _check(lib().qd_int4_gemm_i32(_ptr(aq), M, K, aq.stride(0), _ptr(wp), N, wp.stride(0), _ptr(out),
                                  out.stride(0), _stream(dev)))
    return out


def convrot_w4a4_linear(x, wp, w_scale, bias=None, rotate_block: int = 256, workspace=None, out=None):
    """y = x W^T + b through the rotated INT4 path (quantizer to INT4 codes in
    int8 storage, then the packed-INT4 GEMM with the fused epilogue)."""
    torch = _torch()
    _mat(x, "x"), _mat(wp, "wp")
    dev = _dev(x, wp, w_scale, bias, workspace, out)
    M, K = x.shape
    N = wp.shape[0]
    if wp.shape[1] * 2 != K:
        raise ValueError("wp must be [N, K/2] packed bytes")
    _rows_vec(w_scale, N, torch.float32, "w_scale")
    if bias is not None:
        _rows_vec(bias, N, torch.bfloat16, "bias")
    if workspace is None:
        workspace = torch.empty(max(workspace_size(M, K), 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = _bf16_out(M, N, dev)
    _out(out, (M, N), torch.bfloat16)
    _check(lib().qd_convrot_w4a4_linear(_ptr(x), _dtype_code(x), M, K, x.stride(0), _ptr(wp), N, wp.stride(0),
                                        _ptr(w_scale), _ptr(bias), rotate_block, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0),
                                        _stream(dev)))
    return out
