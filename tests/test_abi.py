"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import quantized_diffusion_amd as qd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdiff.h")

FAKE = ctypes.c_void_p(0x100000)        # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100008)    # 8-byte aligned only
NULL = None
STREAM = ctypes.c_void_p(0)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = qd.lib()
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(L, s), f"{s} declared in qdiff.h but not exported"
    assert set(syms) == set(qd.EXPORTED_SYMBOLS)


def test_version_and_empty_error():
    assert b"gfx950" in qd.lib().qd_version()


def _status(fn, *args):
    st = fn(*args)
    return st, qd.lib().qd_last_error().decode()


Q = qd.QD_BF16


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, Q, -1, 512, 512, 256, FAKE, 512, FAKE, STREAM), qd.QD_EINVAL, "M >= 0"),
    ((FAKE, Q, 4, 0, 512, 256, FAKE, 512, FAKE, STREAM), qd.QD_EINVAL, "K > 0"),
    ((NULL, Q, 4, 512, 512, 256, FAKE, 512, FAKE, STREAM), qd.QD_EINVAL, "null"),
    ((FAKE, Q, 4, 512, 511, 256, FAKE, 512, FAKE, STREAM), qd.QD_EINVAL, "ldx"),
    ((FAKE, Q, 4, 512, 512, 256, FAKE, 500, FAKE, STREAM), qd.QD_EINVAL, "ldq"),
    ((FAKE, Q, 4, 512, 512, 128, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "block"),
    ((FAKE, Q, 4, 528, 528, 256, FAKE, 528, FAKE, STREAM), qd.QD_EUNSUPPORTED, "multiple of the 256"),
    ((FAKE, 7, 4, 512, 512, 256, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "dtype"),
    ((FAKE, Q, 4, 65792, 65792, 256, FAKE, 65792, FAKE, STREAM), qd.QD_EUNSUPPORTED, "exceeds"),
    ((FAKE_ODD, Q, 4, 512, 512, 256, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "aligned"),
    ((FAKE, Q, 4, 512, 516, 256, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "multiples of 16"),
])
def test_quantize_and_rotate_validation(args, status, needle):
    st, msg = _status(qd.lib().qd_quantize_and_rotate_rowwise, *args)
    assert st == status, msg
    assert needle in msg


def test_quantize_rowwise_validation():
    L = qd.lib()
    st, msg = _status(L.qd_quantize_int8_rowwise, FAKE, Q, 4, 24, 24, FAKE, 32, FAKE, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 16" in msg
    st, msg = _status(L.qd_quantize_int8_rowwise, FAKE, Q, 0, 48, 48, FAKE, 48, FAKE, STREAM)
    assert st == qd.QD_OK, msg      # empty problem: nothing enqueued
    st, msg = _status(L.qd_quantize_and_rotate_rowwise_int4, FAKE, Q, 2, 300, 304, 256, FAKE, 304, FAKE, STREAM)
    assert st == qd.QD_EUNSUPPORTED


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, 4, 0, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EINVAL, "K > 0"),
    ((FAKE, 4, 64, 64, FAKE, FAKE, -1, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EINVAL, "N >= 0"),
    ((NULL, 4, 64, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EINVAL, "null"),
    ((FAKE, 4, 64, 32, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EINVAL, "lda"),
    ((FAKE, 4, 64, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 4, STREAM), qd.QD_EINVAL, "leading dimension"),
    ((FAKE, 4, 72, 80, FAKE, FAKE, 8, 80, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EUNSUPPORTED, "multiple of 16"),
    ((FAKE, 4, 64, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 12, STREAM), qd.QD_EUNSUPPORTED, "multiple of 8"),
    ((FAKE_ODD, 4, 64, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EUNSUPPORTED, "aligned"),
    ((FAKE, 4, 64, 72, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EUNSUPPORTED, "multiples of 16"),
    ((FAKE, 4, 64, 64, NULL, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EINVAL, "scale"),
    ((FAKE, 4, 64, 64, FAKE, FAKE, 8, 64, FAKE_ODD, NULL, FAKE, 8, STREAM), qd.QD_EUNSUPPORTED, "w_scale"),
    ((FAKE, 4, 262144, 262144, FAKE, FAKE, 8, 262144, FAKE, NULL, FAKE, 8, STREAM), qd.QD_EUNSUPPORTED, "exceeds"),
    ((FAKE, 0, 64, 64, FAKE, FAKE, 8, 64, FAKE, NULL, FAKE, 8, STREAM), qd.QD_OK, ""),
])
def test_scaled_mm_validation(args, status, needle):
    st, msg = _status(qd.lib().qd_int8_scaled_mm, *args)
    assert st == status, msg
    assert needle in msg


def test_gemm_i32_validation():
    L = qd.lib()
    st, msg = _status(L.qd_int8_gemm_i32, FAKE, 4, 64, 64, FAKE, 4, 64, FAKE, 6, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 4" in msg
    st, msg = _status(L.qd_int8_gemm_i32, FAKE, 4, 64, 64, NULL, 8, 64, FAKE, 8, STREAM)
    assert st == qd.QD_EINVAL


def test_gemm_k_limit():
    """K * 128 * 128 must stay below 2^31 (raw codes include -128): K = 131072
    is refused, the largest accepted K is 131056, on every GEMM entry point."""
    L = qd.lib()
    kmax = int(re.search(r"#define QD_MAX_K_GEMM (\d+)", open(HEADER).read()).group(1))
    assert kmax == 131056 and kmax * 128 * 128 < 2 ** 31 <= (kmax + 16) * 128 * 128
    for K in (131072, 131072 + 64):
        st, msg = _status(L.qd_int8_gemm_i32, FAKE, 4, K, K, FAKE, 8, K, FAKE, 8, STREAM)
        assert st == qd.QD_EUNSUPPORTED and "exceeds" in msg, (K, msg)
        st, msg = _status(L.qd_int8_scaled_mm, FAKE, 4, K, K, FAKE, FAKE, 8, K, FAKE, NULL, FAKE, 8, STREAM)
        assert st == qd.QD_EUNSUPPORTED and "exceeds" in msg, (K, msg)
        st, msg = _status(L.qd_int8_gemm_i32_sliced, FAKE, 4, K, K, 0, FAKE, 8, FAKE, 8, STREAM)
        assert st == qd.QD_EUNSUPPORTED and "exceeds" in msg, (K, msg)
        st, msg = _status(L.qd_int4_gemm_i32, FAKE, 4, K, K, FAKE, 8, K // 2, FAKE, 8, STREAM)
        assert st == qd.QD_EUNSUPPORTED and "exceeds" in msg, (K, msg)
    K6 = 131072   # multiple of 128, above the limit: the FP6 GEMM refuses it too
    st, msg = _status(L.qd_fp6_gemm_i32, FAKE, 4, K6, K6 // 4 * 3, FAKE, 8, K6 // 4 * 3, FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "exceeds" in msg
    # the limit itself passes validation (M = 0: no launch)
    K = kmax
    assert L.qd_int8_gemm_i32(FAKE, 0, K, K, FAKE, 8, K, FAKE, 8, STREAM) == qd.QD_OK
    assert L.qd_int8_scaled_mm(FAKE, 0, K, K, FAKE, FAKE, 8, K, FAKE, NULL, FAKE, 8, STREAM) == qd.QD_OK


def test_gemm_stride_limit():
    """Operand row strides above QD_MAX_LD_GEMM are refused (a tile's copy
    offsets, 384 rows x the stride, must fit 32 bits), and so are output row
    strides above it (store offsets, 160 rows x the stride in bytes); the
    limit passes."""
    L = qd.lib()
    ldmax = int(re.search(r"#define QD_MAX_LD_GEMM (\d+)", open(HEADER).read()).group(1))
    assert ldmax % 16 == 0 and 384 * ldmax < 2 ** 32
    big = ldmax + 16
    K = 256
    cases = [
        (L.qd_int8_gemm_i32, (FAKE, 4, K, big, FAKE, 8, K, FAKE, 8, STREAM)),
        (L.qd_int8_gemm_i32, (FAKE, 4, K, K, FAKE, 8, big, FAKE, 8, STREAM)),
        (L.qd_int8_scaled_mm, (FAKE, 4, K, K, FAKE, FAKE, 8, big, FAKE, NULL, FAKE, 8, STREAM)),
        (L.qd_int4_gemm_i32, (FAKE, 4, K, K, FAKE, 8, big, FAKE, 8, STREAM)),
        (L.qd_int4_gemm_i32, (FAKE, 4, K, big, FAKE, 8, K // 2, FAKE, 8, STREAM)),
        (L.qd_fp6_gemm_i32, (FAKE, 4, K, big, FAKE, 8, K // 4 * 3, FAKE, 8, STREAM)),
        (L.qd_fp6_gemm_i32, (FAKE, 4, K, K // 4 * 3, FAKE, 8, big, FAKE, 8, STREAM)),
        (L.qd_int8_linear, (FAKE, Q, 4, K, K, FAKE, 8, big, FAKE, NULL, 256, FAKE, 1 << 20, FAKE, 8, STREAM)),
        (L.qd_int8_scaled_mm, (FAKE, 4, K, K, FAKE, FAKE, 8, K, FAKE, NULL, FAKE, big, STREAM)),
        (L.qd_int8_gemm_i32, (FAKE, 4, K, K, FAKE, 8, K, FAKE, big, STREAM)),
        (L.qd_fp6_gemm_i32, (FAKE, 4, K, K // 4 * 3, FAKE, 8, K // 4 * 3, FAKE, big, STREAM)),
    ]
    for fn, args in cases:
        st, msg = _status(fn, *args)
        assert st == qd.QD_EUNSUPPORTED and "exceed" in msg, (fn, msg)
    # the limit itself passes validation (M = 0: no launch)
    assert L.qd_int8_gemm_i32(FAKE, 0, K, ldmax, FAKE, 8, ldmax, FAKE, 8, STREAM) == qd.QD_OK
    assert L.qd_fp6_gemm_i32(FAKE, 0, K, ldmax, FAKE, 8, ldmax, FAKE, 8, STREAM) == qd.QD_OK
    assert L.qd_int4_gemm_i32(FAKE, 0, K, K, FAKE, 8, ldmax, FAKE, 8, STREAM) == qd.QD_OK
    assert L.qd_int8_scaled_mm(FAKE, 0, K, K, FAKE, FAKE, 8, K, FAKE, NULL, FAKE, ldmax, STREAM) == qd.QD_OK


def test_linear_validation_and_workspace():
    L = qd.lib()
    M, K, N = 10, 512, 64
    ws = qd.workspace_size(M, K)
    assert ws == 5120 + 256         # codes rounded to 256 B, then the scales
    assert qd.workspace_size(0, K) == 0
    base = dict(x=FAKE, dt=Q, M=M, K=K, ldx=K, wq=FAKE, N=N, ldw=K, sw=FAKE, b=NULL, rb=256,
                ws=FAKE, wsb=ws, y=FAKE, ldy=N, s=STREAM)

    def call(**kw):
        a = dict(base, **kw)
        return _status(L.qd_int8_linear, *a.values())

    assert call(wsb=ws - 1)[0] == qd.QD_EINVAL
    assert call(ws=NULL)[0] == qd.QD_EINVAL
    assert call(ws=ctypes.c_void_p(0x100010))[0] == qd.QD_EUNSUPPORTED
    assert call(rb=128)[0] == qd.QD_EUNSUPPORTED
    assert call(K=528, ldx=528, ldw=528, wsb=10**6)[0] == qd.QD_EUNSUPPORTED
    assert call(rb=0, K=528, ldx=528, ldw=528, wsb=10**6, ldy=60)[0] == qd.QD_EINVAL
    assert call(sw=NULL)[0] == qd.QD_EINVAL
    assert call(b=ctypes.c_void_p(0x100004))[0] == qd.QD_EUNSUPPORTED   # bias must be 8-byte aligned
    assert call(M=0)[0] == qd.QD_OK
    assert call(dt=9)[0] == qd.QD_EUNSUPPORTED


def test_dequantize_validation():
    L = qd.lib()
    st, msg = _status(L.qd_dequantize_int8, FAKE, 4, 40, 48, FAKE, 1, qd.QD_F32, FAKE, 48, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 16" in msg
    st, msg = _status(L.qd_dequantize_int8, FAKE, 4, 48, 48, FAKE, 1, qd.QD_F16, FAKE, 48, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "dtype" in msg
    st, msg = _status(L.qd_dequantize_int8, FAKE, 4, 48, 40, FAKE, 1, qd.QD_F32, FAKE, 48, STREAM)
    assert st == qd.QD_EINVAL
    st, msg = _status(L.qd_dequantize_int8, FAKE, 0, 48, 48, FAKE, 1, qd.QD_F32, FAKE, 48, STREAM)
    assert st == qd.QD_OK


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        qd.quantize_and_rotate_rowwise(torch.zeros(4, 256, dtype=torch.bfloat16))


def test_w4a4_validation():
    L = qd.lib()
    st, msg = _status(L.qd_pack_int4, FAKE, 4, 48, 48, FAKE, 32, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 32" in msg
    st, msg = _status(L.qd_pack_int4, FAKE, 4, 64, 64, FAKE, 16, STREAM)
    assert st == qd.QD_EINVAL
    st, msg = _status(L.qd_int4_scaled_mm, FAKE, 4, 96, 96, FAKE, FAKE, 8, 48, FAKE, NULL, FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 64" in msg
    st, msg = _status(L.qd_int4_scaled_mm, FAKE, 4, 128, 128, FAKE, FAKE, 8, 48, FAKE, NULL, FAKE, 8, STREAM)
    assert st == qd.QD_EINVAL and "K/2" in msg
    st, msg = _status(L.qd_int4_gemm_i32, FAKE, 4, 128, 128, FAKE, 8, 72, FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 16" in msg
    ws = qd.workspace_size(4, 512)
    st, msg = _status(L.qd_convrot_w4a4_linear, FAKE, Q, 4, 512, 512, FAKE, 8, 256, FAKE, NULL, 0, FAKE, ws,
                      FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "rotate_block" in msg
    st, msg = _status(L.qd_convrot_w4a4_linear, FAKE, Q, 0, 512, 512, FAKE, 8, 256, FAKE, NULL, 256, FAKE, ws,
                      FAKE, 8, STREAM)
    assert st == qd.QD_OK


def test_tensorwise_validation():
    L = qd.lib()
    ws = L.qd_quantize_tensorwise_workspace_size()
    assert ws >= 4 * 256
    ok_args = (FAKE, Q, 4, 512, 512, FAKE, 512, FAKE, FAKE, ws, STREAM)
    cases = [
        ((FAKE, Q, 4, 512, 512, FAKE, 512, FAKE, NULL, ws, STREAM), qd.QD_EINVAL, "workspace"),
        ((FAKE, Q, 4, 512, 512, FAKE, 512, FAKE, FAKE, ws - 4, STREAM), qd.QD_EINVAL, "too small"),
        ((FAKE, Q, 4, 520, 520, FAKE, 520, FAKE, FAKE, ws, STREAM), qd.QD_EUNSUPPORTED, "multiple of 16"),
        ((FAKE, Q, 4, 512, 512, NULL, 512, FAKE, FAKE, ws, STREAM), qd.QD_EINVAL, "null"),
        ((FAKE, Q, 4, 512, 512, FAKE, 512, FAKE, ctypes.c_void_p(0x100002), ws, STREAM), qd.QD_EUNSUPPORTED,
         "4-byte"),
    ]
    for args, status, needle in cases:
        st, msg = _status(L.qd_quantize_int8_tensorwise, *args)
        assert st == status and needle in msg, (args, st, msg)
    # M == 0 is a no-op that launches nothing
    assert L.qd_quantize_int8_tensorwise(FAKE, Q, 0, 512, 512, FAKE, 512, FAKE, FAKE, ws, STREAM) == qd.QD_OK
    assert ok_args  # the valid form is exercised on the GPU


def test_scaled_mm_ex_validation():
    L = qd.lib()
    base = dict(aq=FAKE, M=8, K=64, lda=64, a_scale=FAKE, a_len=8, wq=FAKE, N=16, ldw=64, w_scale=FAKE,
                w_len=16, bias=NULL, y=FAKE, ldy=16, s=STREAM)

    def call(**kw):
        a = dict(base, **kw)
        return _status(L.qd_int8_scaled_mm_ex, a["aq"], a["M"], a["K"], a["lda"], a["a_scale"], a["a_len"],
                       a["wq"], a["N"], a["ldw"], a["w_scale"], a["w_len"], a["bias"], a["y"], a["ldy"], a["s"])
    for kw, status, needle in [
        (dict(a_len=3), qd.QD_EINVAL, "a_scale_len"),
        (dict(w_len=2), qd.QD_EINVAL, "w_scale_len"),
        (dict(a_scale=NULL), qd.QD_EINVAL, "null scale"),
        (dict(w_scale=FAKE_ODD), qd.QD_EUNSUPPORTED, "16-byte"),
        (dict(K=40, lda=40, ldw=40), qd.QD_EUNSUPPORTED, "multiple of 16"),
    ]:
        st, msg = call(**kw)
        assert st == status and needle in msg, (kw, st, msg)
    # a per-tensor w_scale needs no 16-byte alignment: validation passes up to the launch,
    # which an empty problem skips
    assert call(w_len=1, w_scale=ctypes.c_void_p(0x100004), M=0)[0] == qd.QD_OK


def test_act_validation():
    L = qd.lib()
    F16, F32 = qd.QD_F16, qd.QD_F32
    # quantizer with an activation
    for args, status, needle in [
        ((FAKE, F32, 4, 512, 512, 1, 256, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "BF16 or FP16"),
        ((FAKE, Q, 4, 512, 512, 9, 256, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "unknown activation"),
        ((FAKE, Q, 4, 33024, 33024, 1, 256, FAKE, 33024, FAKE, STREAM), qd.QD_EUNSUPPORTED, "32768"),
        ((FAKE, Q, 4, 512, 512, 1, 128, FAKE, 512, FAKE, STREAM), qd.QD_EUNSUPPORTED, "rotate_block"),
    ]:
        st, msg = _status(L.qd_quantize_rowwise_act, *args)
        assert st == status and needle in msg, (args, st, msg)
    # ReLU has no FP64 temporaries: long rows are fine (M == 0 stops before any launch)
    assert L.qd_quantize_rowwise_act(FAKE, F16, 0, 65536, 65536, 4, 256, FAKE, 65536, FAKE, STREAM) == qd.QD_OK
    # the layer
    st, msg = _status(L.qd_int8_linear_act, FAKE, F32, 4, 512, 512, 3, FAKE, 8, 512, FAKE, NULL, 256,
                      FAKE, 1 << 20, FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "BF16 or FP16" in msg
    # the elementwise entry
    for args, status, needle in [
        ((FAKE, F32, 16, 1, FAKE, STREAM), qd.QD_EUNSUPPORTED, "BF16 or FP16"),
        ((FAKE, Q, -1, 1, FAKE, STREAM), qd.QD_EINVAL, "n >= 0"),
        ((NULL, Q, 16, 1, FAKE, STREAM), qd.QD_EINVAL, "null"),
        ((ctypes.c_void_p(0x100001), Q, 16, 1, FAKE, STREAM), qd.QD_EUNSUPPORTED, "2-byte"),
        ((FAKE, Q, 16, 7, FAKE, STREAM), qd.QD_EUNSUPPORTED, "unknown activation"),
    ]:
        st, msg = _status(L.qd_input_act, *args)
        assert st == status and needle in msg, (args, st, msg)


def test_fp6_validation():
    L = qd.lib()
    # fused FP6 quantizer: 16-bit input only, ld6 >= 3K/4 and a multiple of 16
    for args, status, needle in [
        ((FAKE, qd.QD_F32, 4, 512, 512, 256, FAKE, 384, FAKE, STREAM), qd.QD_EUNSUPPORTED, "BF16 or FP16"),
        ((FAKE, Q, 4, 512, 512, 256, FAKE, 368, FAKE, STREAM), qd.QD_EINVAL, "ldq"),
        ((FAKE, Q, 4, 512, 512, 256, FAKE, 392, FAKE, STREAM), qd.QD_EUNSUPPORTED, "multiples of 16"),
        ((FAKE, Q, 4, 640, 640, 256, FAKE, 480, FAKE, STREAM), qd.QD_EUNSUPPORTED, "256"),
    ]:
        st, msg = _status(L.qd_quantize_and_rotate_rowwise_fp6, *args)
        assert st == status and needle in msg, (args, st, msg)
    assert L.qd_quantize_and_rotate_rowwise_fp6(FAKE, Q, 0, 512, 512, 256, FAKE, 384, FAKE, STREAM) == qd.QD_OK
    # packing and the FP6 GEMM
    st, msg = _status(L.qd_pack_fp6, FAKE, 4, 96, 96, FAKE, 80, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 64" in msg
    st, msg = _status(L.qd_pack_fp6, FAKE, 4, 128, 128, FAKE, 80, STREAM)
    assert st == qd.QD_EINVAL and "3K/4" in msg
    st, msg = _status(L.qd_fp6_scaled_mm, FAKE, 8, 192, 144, FAKE, FAKE, 8, 144, FAKE, NULL, FAKE, 8, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 128" in msg
    st, msg = _status(L.qd_fp6_scaled_mm, FAKE, 8, 256, 176, FAKE, FAKE, 8, 192, FAKE, NULL, FAKE, 8, STREAM)
    assert st == qd.QD_EINVAL and "3K/4" in msg
    st, msg = _status(L.qd_fp6_gemm_i32, FAKE, 8, 256, 192, FAKE, 8, 192, FAKE, 10, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "multiple of 4" in msg


def test_gemm_tiles_setting():
    L = qd.lib()
    for bad in (-1, 3, 99):
        assert L.qd_set_gemm_tiles(bad) == qd.QD_EINVAL
        assert b"tile setting" in L.qd_last_error()
    for good in (qd.GEMM_TILES_256x384, qd.GEMM_TILES_256x256, qd.GEMM_TILES_AUTO):
        assert L.qd_set_gemm_tiles(good) == qd.QD_OK
    with pytest.raises(qd.QDiffError):
        qd.set_gemm_tiles(7)
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)


def test_gemm_tiles_choice():
    """The shape rule: rounds of 256 workgroups, a wide round costing 1.41x."""
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)
    assert qd.int8_gemm_tiles(32700, 16128, 5376) == qd.GEMM_TILES_256x384   # 32 vs 21 rounds
    assert qd.int8_gemm_tiles(14850, 28672, 7168) == qd.GEMM_TILES_256x384   # 26 vs 18
    assert qd.int8_gemm_tiles(1000, 1000, 320) == qd.GEMM_TILES_256x256      # one round either way
    assert qd.int8_gemm_tiles(32700, 16128, 5392) == qd.GEMM_TILES_256x256   # K % 64 != 0: general kernel
    qd.set_gemm_tiles(qd.GEMM_TILES_256x384)
    assert qd.int8_gemm_tiles(1000, 1000, 320) == qd.GEMM_TILES_256x384
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)


def test_attention_validation():
    L = qd.lib()
    ws = qd.attention_workspace_size(2, 100, 70, 128)
    assert ws >= 2 * 100 * 128 + 2 * 2 * 70 * 128 + 4 * 2 * (100 + 2 * 70)
    assert qd.attention_workspace_size(0, 1, 1, 64) == 0
    A = ctypes.c_void_p(0x100000)
    big = ctypes.c_size_t(1 << 40)
    args = lambda BH, Lq, Lk, D, ws_ptr=A, n=big, q=A: (q, A, A, qd.QD_BF16, BH, Lq, Lk, D, ctypes.c_float(0.0),
                                                        ws_ptr, n, A, STREAM)
    assert L.qd_int8_attention(*args(1, 4, 4, 96)) == qd.QD_EUNSUPPORTED
    assert b"head dim" in L.qd_last_error()
    assert L.qd_int8_attention(*args(0, 4, 4, 64)) == qd.QD_EINVAL
    assert L.qd_int8_attention(*args(1, 4, 0, 64)) == qd.QD_EINVAL
    assert L.qd_int8_attention(*args(70000, 4, 4, 64)) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_attention(*args(1, 0, 4, 64)) == qd.QD_OK          # nothing to do
    assert L.qd_int8_attention(*args(1, 4, 4, 64, n=ctypes.c_size_t(16))) == qd.QD_EINVAL
    assert b"workspace too small" in L.qd_last_error()
    assert L.qd_int8_attention(*args(1, 4, 4, 64, ws_ptr=ctypes.c_void_p(0x100010))) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_attention(*args(1, 4, 4, 64, q=FAKE_ODD)) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_attention(*args(1, 4, 4, 64, q=NULL)) == qd.QD_EINVAL


def test_attention_codes_validation():
    L = qd.lib()
    A = ctypes.c_void_p(0x100000)
    f = lambda BH, Lq, Lk, D, qc=A, s=A: L.qd_int8_attention_codes(qc, s, A, A, A, A, BH, Lq, Lk, D,
                                                                   ctypes.c_float(0.0), A, STREAM)
    assert f(1, 4, 4, 32) == qd.QD_EUNSUPPORTED
    assert f(1, 4, 0, 64) == qd.QD_EINVAL
    assert f(1, 0, 4, 64) == qd.QD_OK
    assert f(1, 4, 4, 64, qc=FAKE_ODD) == qd.QD_EUNSUPPORTED
    assert f(1, 4, 4, 64, s=ctypes.c_void_p(0x100002)) == qd.QD_EUNSUPPORTED
    assert f(1, 4, 4, 64, qc=NULL) == qd.QD_EINVAL


def test_sliced_weights_validation():
    """K-sliced weight entry points: argument checks before any device work."""
    L = qd.lib()
    A = FAKE
    ws = ctypes.c_size_t(1 << 30)
    # slicing: K % 64, ldw >= K, alignment, nulls, empty
    assert L.qd_int8_slice_weights(A, 8, 96, 96, A, STREAM) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_slice_weights(A, 8, 128, 64, A, STREAM) == qd.QD_EINVAL
    assert L.qd_int8_slice_weights(NULL, 8, 128, 128, A, STREAM) == qd.QD_EINVAL
    assert L.qd_int8_slice_weights(FAKE_ODD, 8, 128, 128, A, STREAM) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_slice_weights(A, 8, 128, 136, A, STREAM) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_slice_weights(NULL, 0, 128, 128, NULL, STREAM) == qd.QD_OK
    assert L.qd_int8_slice_weights(A, -1, 128, 128, A, STREAM) == qd.QD_EINVAL
    # GEMMs: K % 64 (K % 16 alone is not enough for the sliced layout)
    for a_sl in (0, 1):
        assert L.qd_int8_scaled_mm_sliced(A, 4, 96, 96, a_sl, A, A, 8, A, NULL, A, 8, STREAM) == qd.QD_EUNSUPPORTED
        assert L.qd_int8_gemm_i32_sliced(A, 4, 96, 96, a_sl, A, 8, A, 8, STREAM) == qd.QD_EUNSUPPORTED
        assert L.qd_int8_scaled_mm_sliced(A, 4, 128, 128, a_sl, NULL, A, 8, A, NULL, A, 8, STREAM) == qd.QD_EINVAL
        assert L.qd_int8_gemm_i32_sliced(A, 4, 128, 128, a_sl, FAKE_ODD, 8, A, 8, STREAM) == qd.QD_EUNSUPPORTED
        assert L.qd_int8_gemm_i32_sliced(A, 0, 128, 128, a_sl, A, 8, A, 8, STREAM) == qd.QD_OK
    # lda matters for row-major codes only
    assert L.qd_int8_gemm_i32_sliced(A, 4, 128, 64, 0, A, 8, A, 8, STREAM) == qd.QD_EINVAL
    # the sliced quantizer: rotation block 256, K % 256
    q = lambda K, blk=256, x=A, dt=qd.QD_BF16, act=qd.ACT_NONE: L.qd_quantize_and_rotate_rowwise_sliced(
        x, dt, 4, K, K, act, blk, A, A, STREAM)
    assert q(320) == qd.QD_EUNSUPPORTED
    assert q(512, blk=0) == qd.QD_EUNSUPPORTED
    assert q(512, x=NULL) == qd.QD_EINVAL
    assert q(512, x=FAKE_ODD) == qd.QD_EUNSUPPORTED
    assert q(512, dt=qd.QD_F32, act=qd.ACT_SILU) == qd.QD_EUNSUPPORTED
    assert q(512, act=7) == qd.QD_EUNSUPPORTED
    assert L.qd_quantize_and_rotate_rowwise_sliced(A, qd.QD_BF16, 0, 512, 512, 0, 256, A, A, STREAM) == qd.QD_OK
    # the layer: K % 64 with or without rotation, then the usual checks
    f = lambda K, rb, x=A, w=A, act=qd.ACT_NONE: L.qd_int8_linear_sliced(
        x, qd.QD_BF16, 4, K, K, act, w, 8, A, NULL, rb, ctypes.c_void_p(0x100000), ws, A, 8, STREAM)
    assert f(96, 0) == qd.QD_EUNSUPPORTED
    assert f(320, 256) == qd.QD_EUNSUPPORTED
    assert f(128, 128) == qd.QD_EUNSUPPORTED
    assert f(128, 0, w=NULL) == qd.QD_EINVAL
    assert f(128, 0, x=FAKE_ODD) == qd.QD_EUNSUPPORTED
    assert f(128, 0, act=9) == qd.QD_EUNSUPPORTED
    assert L.qd_int8_linear_sliced(A, qd.QD_BF16, 0, 128, 128, qd.ACT_NONE, A, 8, A, NULL, 0, NULL, ctypes.c_size_t(0),
                                   A, 8, STREAM) == qd.QD_OK


def test_sliced_python_shape_checks():
    """The binding's layout checks reject anything but an int8 [K / 64, N, 64] tensor (CPU tensors suffice)."""
    import torch

    with pytest.raises(ValueError):
        qd._sliced(torch.zeros(4, 8, 32, dtype=torch.int8))
    with pytest.raises(ValueError):
        qd._sliced(torch.zeros(4, 8, 64, dtype=torch.uint8))
    with pytest.raises(ValueError):
        qd._sliced(torch.zeros(8, 4, 64, dtype=torch.int8).transpose(0, 1))
    assert qd._sliced(torch.zeros(3, 5, 64, dtype=torch.int8)) == (192, 5)


def test_fp6_sliced_validation():
    """K-sliced FP6 entry points: argument checks before any device work."""
    L = qd.lib()
    A = FAKE
    ws = ctypes.c_size_t(1 << 30)
    assert L.qd_fp6_slice_weights(A, 8, 192, 144, A, STREAM) == qd.QD_EUNSUPPORTED      # K % 128
    assert L.qd_fp6_slice_weights(A, 8, 256, 96, A, STREAM) == qd.QD_EINVAL             # ldw < 3K/4
    assert L.qd_fp6_slice_weights(NULL, 8, 256, 192, A, STREAM) == qd.QD_EINVAL
    assert L.qd_fp6_slice_weights(FAKE_ODD, 8, 256, 192, A, STREAM) == qd.QD_EUNSUPPORTED
    assert L.qd_fp6_slice_weights(NULL, 0, 256, 192, NULL, STREAM) == qd.QD_OK
    q = lambda K, dt=qd.QD_BF16, blk=256: L.qd_quantize_and_rotate_rowwise_fp6_sliced(A, dt, 4, K, K, blk, A, A, STREAM)
    assert q(512, dt=qd.QD_F32) == qd.QD_EUNSUPPORTED
    assert q(384) == qd.QD_EUNSUPPORTED                                                  # K % 256 for the rotation
    assert q(512, blk=0) == qd.QD_EUNSUPPORTED
    for a_sl in (0, 1):
        assert L.qd_fp6_gemm_i32_sliced(A, 4, 192, 144, a_sl, A, 8, A, 8, STREAM) == qd.QD_EUNSUPPORTED
        assert L.qd_fp6_gemm_i32_sliced(A, 0, 256, 192, a_sl, A, 8, A, 8, STREAM) == qd.QD_OK
        assert L.qd_fp6_scaled_mm_sliced(A, 4, 256, 192, a_sl, NULL, A, 8, A, NULL, A, 8, STREAM) == qd.QD_EINVAL
    assert L.qd_fp6_gemm_i32_sliced(A, 4, 256, 96, 0, A, 8, A, 8, STREAM) == qd.QD_EINVAL  # lda < 3K/4 (row-major a6)
    f = lambda dt, K=512, rb=256: L.qd_convrot_w4a4_linear_fp6_sliced(A, dt, 4, K, K, A, 8, A, NULL, rb,
                                                                    ctypes.c_void_p(0x100000), ws, A, 8, STREAM)
    assert f(qd.QD_F32) == qd.QD_EUNSUPPORTED
    assert f(qd.QD_BF16, rb=0) == qd.QD_EUNSUPPORTED
    assert f(qd.QD_BF16, K=384) == qd.QD_EUNSUPPORTED


def test_output_tensor_checks():
    """Caller-provided outputs are checked for dtype and exact shape (the kernels
    write the whole extent), so a short buffer raises instead of being overrun."""
    import torch

    qd._out(torch.empty(4, 8, dtype=torch.bfloat16), (4, 8), torch.bfloat16)
    qd._out(torch.empty(4, 16, dtype=torch.bfloat16)[:, :8], (4, 8), torch.bfloat16)   # padded rows are fine
    with pytest.raises(ValueError):
        qd._out(torch.empty(3, 8, dtype=torch.bfloat16), (4, 8), torch.bfloat16)
    with pytest.raises(ValueError):
        qd._out(torch.empty(4, 8, dtype=torch.float32), (4, 8), torch.bfloat16)
    with pytest.raises(ValueError):
        qd._out(torch.empty(8, 4, dtype=torch.bfloat16).t(), (4, 8), torch.bfloat16)
    with pytest.raises(ValueError):
        qd._out(torch.empty(2, 4, 8, 64, dtype=torch.int8)[:, 0], (2, 8, 64), torch.int8)
    qd._out(torch.empty(2, 8, 64, dtype=torch.int8), (2, 8, 64), torch.int8)
    with pytest.raises(ValueError):
        qd._f6_rows(torch.empty(4, 90, dtype=torch.uint8), 128, "a6")
    qd._f6_rows(torch.empty(4, 96, dtype=torch.uint8), 128, "a6")


def test_tensorwise_noalloc_validation():
    """The allocation-free tensor-wise entry point checks its arguments as the
    workspace entry point does, before any HIP call."""
    L = qd.lib()
    f = L.qd_quantize_int8_tensorwise_noalloc
    assert f(FAKE, Q, 0, 512, 512, FAKE, 512, FAKE, STREAM) == qd.QD_OK           # empty: nothing to do
    st, msg = _status(f, NULL, Q, 4, 512, 512, FAKE, 512, FAKE, STREAM)
    assert st == qd.QD_EINVAL and "null" in msg
    st, msg = _status(f, FAKE, Q, 4, 40, 40, FAKE, 48, FAKE, STREAM)
    assert st == qd.QD_EUNSUPPORTED
    st, msg = _status(f, FAKE, Q, 4, 512, 500, FAKE, 512, FAKE, STREAM)
    assert st == qd.QD_EINVAL
    st, msg = _status(f, FAKE_ODD, Q, 4, 512, 512, FAKE, 512, FAKE, STREAM)
    assert st == qd.QD_EUNSUPPORTED and "aligned" in msg


def test_gemm_tiles_setting_is_per_thread():
    """A thread's tile setting does not change the tiles another thread's launches use."""
    import threading
    L = qd.lib()
    shape = (32700, 16128, 5376)
    auto = L.qd_int8_gemm_tiles(*shape)
    assert L.qd_set_gemm_tiles(qd.GEMM_TILES_256x256) == qd.QD_OK
    try:
        seen = {}
        t = threading.Thread(target=lambda: seen.update(other=L.qd_int8_gemm_tiles(*shape)))
        t.start()
        t.join()
        assert seen["other"] == auto                                   # the other thread: still automatic
        assert L.qd_int8_gemm_tiles(*shape) == qd.GEMM_TILES_256x256   # this thread: fixed
    finally:
        L.qd_set_gemm_tiles(qd.GEMM_TILES_AUTO)
