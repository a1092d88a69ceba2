// C ABI of the library (declared in include/qdiff.h): argument validation on
// the host, then kernel launches on the caller's stream.  Nothing here
// allocates, frees or synchronises, and no C++ exception crosses the ABI.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/qdiff.h"
#include "qd_launch.h"

namespace {

thread_local char g_err[512] = "";

qd_status_t fail(qd_status_t st, const char* fn, const char* fmt, ...) {
    int n = snprintf(g_err, sizeof(g_err), "%s: ", fn);
    if (n < 0) n = 0;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err + n, sizeof(g_err) - (size_t)n, fmt, ap);
    va_end(ap);
    return st;
}

qd_status_t ok() {
    g_err[0] = '\0';
    return QD_OK;
}

qd_status_t hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(QD_EHIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int dtype_size(qd_dtype_t dt) { return dt == QD_F32 ? 4 : 2; }

bool dtype_ok(qd_dtype_t dt) { return dt == QD_F32 || dt == QD_BF16 || dt == QD_F16; }

// Shared checks of the quantizers.
// min_ldq: smallest row stride of q in bytes (K for one code per byte).
qd_status_t check_quant(const char* fn, const void* x, qd_dtype_t dt, int64_t M, int64_t K,
                        int64_t ldx, bool rotate, int32_t block, const int8_t* q, int64_t ldq,
                        const float* scale, int64_t min_ldq = -1) {
    if (M < 0 || K <= 0) return fail(QD_EINVAL, fn, "need M >= 0 and K > 0 (M=%lld, K=%lld)", (long long)M, (long long)K);
    if (M > 0 && (!x || !q || !scale)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (!dtype_ok(dt)) return fail(QD_EUNSUPPORTED, fn, "unknown input dtype %d", (int)dt);
    if (ldx < K) return fail(QD_EINVAL, fn, "ldx (%lld) < K (%lld)", (long long)ldx, (long long)K);
    if (min_ldq < 0) min_ldq = K;
    if (ldq < min_ldq) return fail(QD_EINVAL, fn, "ldq (%lld) < %lld", (long long)ldq, (long long)min_ldq);
    if (rotate && block != 256) return fail(QD_EUNSUPPORTED, fn, "rotation block must be 256 (got %d)", block);
    if (rotate && K % 256 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of the 256-wide rotation block", (long long)K);
    if (K % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 16", (long long)K);
    if (K > QD_MAX_K_QUANT) return fail(QD_EUNSUPPORTED, fn, "K (%lld) exceeds %d", (long long)K, QD_MAX_K_QUANT);
    if (M > INT32_MAX) return fail(QD_EUNSUPPORTED, fn, "M (%lld) exceeds INT32_MAX", (long long)M);
    if (M > 0 && (!aligned16(x) || !aligned16(q)))
        return fail(QD_EUNSUPPORTED, fn, "x and q must be 16-byte aligned");
    if ((ldx * dtype_size(dt)) % 16 != 0 || ldq % 16 != 0)
        return fail(QD_EUNSUPPORTED, fn, "row strides must be multiples of 16 bytes (ldx*%d=%lld, ldq=%lld)",
                    dtype_size(dt), (long long)(ldx * dtype_size(dt)), (long long)ldq);
    return QD_OK;
}

qd_status_t check_gemm(const char* fn, const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                       const int8_t* wq, int64_t N, int64_t ldw, const void* out, int64_t ldo,
                       int64_t ldo_multiple) {
    if (M < 0 || N < 0 || K <= 0)
        return fail(QD_EINVAL, fn, "need M >= 0, N >= 0, K > 0 (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N, (long long)K);
    if (M > 0 && N > 0 && (!aq || !wq || !out)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (lda < K || ldw < K) return fail(QD_EINVAL, fn, "lda/ldw must be >= K");
    if (lda > QD_MAX_LD_GEMM || ldw > QD_MAX_LD_GEMM)
        return fail(QD_EUNSUPPORTED, fn, "lda/ldw (%lld, %lld) exceed %d", (long long)lda, (long long)ldw, QD_MAX_LD_GEMM);
    if (ldo < N) return fail(QD_EINVAL, fn, "output leading dimension (%lld) < N (%lld)", (long long)ldo, (long long)N);
    if (ldo > QD_MAX_LD_GEMM)
        return fail(QD_EUNSUPPORTED, fn, "output leading dimension (%lld) exceeds %d", (long long)ldo, QD_MAX_LD_GEMM);
    if (K % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 16", (long long)K);
    if (K > QD_MAX_K_GEMM) return fail(QD_EUNSUPPORTED, fn, "K (%lld) exceeds %d", (long long)K, QD_MAX_K_GEMM);
    if (M > INT32_MAX - 256 || N > INT32_MAX - 256) return fail(QD_EUNSUPPORTED, fn, "M or N too large");
    if ((M + 255) / 256 * ((N + 255) / 256) > INT32_MAX)
        return fail(QD_EUNSUPPORTED, fn, "too many output tiles");
    if (M > 0 && N > 0 && (!aligned16(aq) || !aligned16(wq) || !aligned16(out)))
        return fail(QD_EUNSUPPORTED, fn, "aq, wq and the output must be 16-byte aligned");
    if (lda % 16 != 0 || ldw % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "lda and ldw must be multiples of 16");
    if (ldo % ldo_multiple != 0)
        return fail(QD_EUNSUPPORTED, fn, "output leading dimension must be a multiple of %lld", (long long)ldo_multiple);
    return QD_OK;
}

// An input activation needs a 16-bit input (the activation's result is
// rounded to that type); the FP64 activations allow rows of up to 32768.
qd_status_t check_act(const char* fn, qd_act_t act, qd_dtype_t dt, int64_t K) {
    if ((int)act < (int)QD_ACT_NONE || (int)act > (int)QD_ACT_RELU)
        return fail(QD_EUNSUPPORTED, fn, "unknown activation %d", (int)act);
    if (act == QD_ACT_NONE) return QD_OK;
    if (dt != QD_BF16 && dt != QD_F16)
        return fail(QD_EUNSUPPORTED, fn, "an input activation needs a BF16 or FP16 input");
    if (act != QD_ACT_RELU && K > 32768)
        return fail(QD_EUNSUPPORTED, fn, "K (%lld) exceeds 32768 with this activation", (long long)K);
    return QD_OK;
}

qd_status_t quantize_impl(const char* fn, const void* x, qd_dtype_t dt, int64_t M, int64_t K,
                          int64_t ldx, bool rotate, int32_t block, int qmax, int8_t* q,
                          int64_t ldq, float* scale, hipStream_t stream, qd_act_t act = QD_ACT_NONE) {
    qd_status_t st = check_quant(fn, x, dt, M, K, ldx, rotate, block, q, ldq, scale);
    if (st != QD_OK) return st;
    st = check_act(fn, act, dt, K);
    if (st != QD_OK) return st;
    if (M == 0) return ok();
    return hip_status(fn, qd::launch_rotquant(x, (int)dt, rotate, qmax, M, K, ldx, q, ldq, scale, stream,
                                              (int)act));
}

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t ws_codes_bytes(int64_t M, int64_t K) { return round_up((size_t)M * (size_t)round_up((size_t)K, 16), kAlign); }

}  // namespace

extern "C" {

const char* qd_last_error(void) { return g_err; }

const char* qd_version(void) { return "qdiff 0.1.0 (gfx950)"; }

qd_status_t qd_quantize_and_rotate_rowwise(const void* x, qd_dtype_t x_dtype, int64_t M,
                                           int64_t K, int64_t ldx, int32_t block, int8_t* q,
                                           int64_t ldq, float* row_scale, hipStream_t stream) {
    return quantize_impl("qd_quantize_and_rotate_rowwise", x, x_dtype, M, K, ldx, true, block, 127,
                         q, ldq, row_scale, stream);
}

qd_status_t qd_quantize_and_rotate_rowwise_int4(const void* x, qd_dtype_t x_dtype, int64_t M,
                                                int64_t K, int64_t ldx, int32_t block,
                                                int8_t* q, int64_t ldq, float* row_scale,
                                                hipStream_t stream) {
    return quantize_impl("qd_quantize_and_rotate_rowwise_int4", x, x_dtype, M, K, ldx, true, block,
                         7, q, ldq, row_scale, stream);
}

qd_status_t qd_quantize_int8_rowwise(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                     int64_t ldx, int8_t* q, int64_t ldq, float* row_scale,
                                     hipStream_t stream) {
    return quantize_impl("qd_quantize_int8_rowwise", x, x_dtype, M, K, ldx, false, 0, 127, q, ldq,
                         row_scale, stream);
}

qd_status_t qd_int8_scaled_mm(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                              const float* a_scale, const int8_t* wq, int64_t N, int64_t ldw,
                              const float* w_scale, const void* bias_bf16, void* y_bf16,
                              int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_int8_scaled_mm";
    qd_status_t st = check_gemm(fn, aq, M, K, lda, wq, N, ldw, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_bf16(aq, lda, a_scale, wq, ldw, w_scale, bias_bf16,
                                               y_bf16, ldy, M, N, K, stream));
}

qd_status_t qd_int8_scaled_mm_sliced(const int8_t* aq, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                     const float* a_scale, const int8_t* w_sliced, int64_t N,
                                     const float* w_scale, const void* bias_bf16, void* y_bf16,
                                     int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_int8_scaled_mm_sliced";
    if (K % 64 != 0) return fail(QD_EUNSUPPORTED, fn, "K-sliced weights need K %% 64 == 0 (K=%lld)", (long long)K);
    qd_status_t st = check_gemm(fn, aq, M, K, a_sliced ? K : lda, w_sliced, N, K, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_bf16(aq, lda, a_scale, w_sliced, K, w_scale, bias_bf16, y_bf16, ldy,
                                               M, N, K, stream, 1, 1, true, a_sliced != 0));
}

qd_status_t qd_quantize_and_rotate_rowwise_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                  int64_t ldx, qd_act_t input_act, int32_t block,
                                                  int8_t* q_sliced, float* row_scale, hipStream_t stream) {
    const char* fn = "qd_quantize_and_rotate_rowwise_sliced";
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, true, block, q_sliced, K, row_scale);
    if (st != QD_OK) return st;
    st = check_act(fn, input_act, x_dtype, K);
    if (st != QD_OK) return st;
    if (M == 0) return ok();
    return hip_status(fn, qd::launch_rotquant_sliced(x, (int)x_dtype, M, K, ldx, q_sliced, row_scale, stream,
                                                     (int)input_act));
}

qd_status_t qd_int8_scaled_mm_ex(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                                 const float* a_scale, int64_t a_scale_len, const int8_t* wq,
                                 int64_t N, int64_t ldw, const float* w_scale, int64_t w_scale_len,
                                 const void* bias_bf16, void* y_bf16, int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_int8_scaled_mm_ex";
    qd_status_t st = check_gemm(fn, aq, M, K, lda, wq, N, ldw, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (a_scale_len != M && a_scale_len != 1)
        return fail(QD_EINVAL, fn, "a_scale_len must be M (%lld) or 1 (got %lld)", (long long)M, (long long)a_scale_len);
    if (w_scale_len != N && w_scale_len != 1)
        return fail(QD_EINVAL, fn, "w_scale_len must be N (%lld) or 1 (got %lld)", (long long)N, (long long)w_scale_len);
    const int a_step = a_scale_len == M ? 1 : 0;
    const int w_step = w_scale_len == N ? 1 : 0;
    if ((w_step && ((uintptr_t)w_scale & 15u)) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "a per-channel w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_bf16(aq, lda, a_scale, wq, ldw, w_scale, bias_bf16, y_bf16, ldy, M,
                                               N, K, stream, a_step, w_step));
}

size_t qd_quantize_tensorwise_workspace_size(void) { return (size_t)qd::kTensorwisePartials * sizeof(float); }

qd_status_t qd_quantize_int8_tensorwise(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                        int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "qd_quantize_int8_tensorwise";
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, false, 0, q, ldq, scale);
    if (st != QD_OK) return st;
    if (M == 0) return ok();
    if (!workspace) return fail(QD_EINVAL, fn, "null workspace");
    if (workspace_bytes < qd_quantize_tensorwise_workspace_size())
        return fail(QD_EINVAL, fn, "workspace too small (%zu < %zu bytes)", workspace_bytes,
                    qd_quantize_tensorwise_workspace_size());
    if ((uintptr_t)workspace & 3u) return fail(QD_EUNSUPPORTED, fn, "workspace must be 4-byte aligned");
    return hip_status(fn, qd::launch_quant_tensorwise(x, (int)x_dtype, M, K, ldx, q, ldq, scale,
                                                      static_cast<float*>(workspace), stream));
}

qd_status_t qd_quantize_int8_tensorwise_noalloc(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                                hipStream_t stream) {
    const char* fn = "qd_quantize_int8_tensorwise_noalloc";
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, false, 0, q, ldq, scale);
    if (st != QD_OK) return st;
    if (M == 0) return ok();
    float* partial = nullptr;
    size_t cap = 0;
    const hipError_t e = qd::tensorwise_scratch(stream, &partial, &cap);
    if (e != hipSuccess)
        return fail(QD_EHIP, fn, "locating the library's scratch array failed: %s", hipGetErrorString(e));
    // pass 1 writes one partial per workgroup, min(M, kTensorwisePartials) of them
    const int64_t need = M < qd::kTensorwisePartials ? M : qd::kTensorwisePartials;
    if ((size_t)need > cap)
        return fail(QD_EUNSUPPORTED, fn, "%lld partial maxima exceed the %zu-float scratch array", (long long)need, cap);
    return hip_status(fn, qd::launch_quant_tensorwise(x, (int)x_dtype, M, K, ldx, q, ldq, scale, partial, stream));
}

size_t qd_int8_linear_workspace_size(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return ws_codes_bytes(M, K) + round_up((size_t)M * sizeof(float), kAlign);
}

static qd_status_t linear_impl(const char* fn, const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                               int64_t ldx, qd_act_t act, const int8_t* wq, int64_t N, int64_t ldw,
                               const float* w_scale, const void* bias_bf16, int32_t rotate_block,
                               void* workspace, size_t workspace_bytes, void* y_bf16, int64_t ldy,
                               hipStream_t stream, bool w_sliced = false) {
    if (w_sliced && K % 64 != 0)
        return fail(QD_EUNSUPPORTED, fn, "K-sliced weights need K %% 64 == 0 (K=%lld)", (long long)K);
    if (rotate_block != 0 && rotate_block != 256)
        return fail(QD_EUNSUPPORTED, fn, "rotate_block must be 0 or 256 (got %d)", rotate_block);
    const bool rotate = rotate_block == 256;
    if (M < 0 || N < 0 || K <= 0)
        return fail(QD_EINVAL, fn, "need M >= 0, N >= 0, K > 0 (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    const int64_t ldq = (int64_t)round_up((size_t)K, 16);
    if (!workspace) return fail(QD_EINVAL, fn, "null workspace");
    if ((uintptr_t)workspace % kAlign) return fail(QD_EUNSUPPORTED, fn, "workspace must be 256-byte aligned");
    if (workspace_bytes < qd_int8_linear_workspace_size(M, K))
        return fail(QD_EINVAL, fn, "workspace too small: %zu < %zu bytes", workspace_bytes,
                    qd_int8_linear_workspace_size(M, K));
    int8_t* aq = static_cast<int8_t*>(workspace);
    float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_codes_bytes(M, K));
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, rotate, rotate_block, aq, ldq, sx);
    if (st != QD_OK) return st;
    st = check_act(fn, act, x_dtype, K);
    if (st != QD_OK) return st;
    st = check_gemm(fn, aq, M, K, ldq, wq, N, ldw, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (!w_scale) return fail(QD_EINVAL, fn, "null w_scale");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    // with K-sliced weights and rotation, the activation codes go to the workspace K-sliced too
    const bool a_sliced = w_sliced && rotate;
    hipError_t e = a_sliced ? qd::launch_rotquant_sliced(x, (int)x_dtype, M, K, ldx, aq, sx, stream, (int)act)
                            : qd::launch_rotquant(x, (int)x_dtype, rotate, 127, M, K, ldx, aq, ldq, sx, stream,
                                                  (int)act);
    if (e != hipSuccess) return hip_status(fn, e);
    return hip_status(fn, qd::launch_gemm_bf16(aq, ldq, sx, wq, ldw, w_scale, bias_bf16, y_bf16,
                                               ldy, M, N, K, stream, 1, 1, w_sliced, a_sliced));
}

qd_status_t qd_int8_linear(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                           int64_t ldx, const int8_t* wq, int64_t N, int64_t ldw,
                           const float* w_scale, const void* bias_bf16, int32_t rotate_block,
                           void* workspace, size_t workspace_bytes, void* y_bf16, int64_t ldy,
                           hipStream_t stream) {
    return linear_impl("qd_int8_linear", x, x_dtype, M, K, ldx, QD_ACT_NONE, wq, N, ldw, w_scale, bias_bf16,
                       rotate_block, workspace, workspace_bytes, y_bf16, ldy, stream);
}

qd_status_t qd_int8_linear_act(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                               qd_act_t input_act, const int8_t* wq, int64_t N, int64_t ldw,
                               const float* w_scale, const void* bias_bf16, int32_t rotate_block,
                               void* workspace, size_t workspace_bytes, void* y_bf16, int64_t ldy,
                               hipStream_t stream) {
    return linear_impl("qd_int8_linear_act", x, x_dtype, M, K, ldx, input_act, wq, N, ldw, w_scale, bias_bf16,
                       rotate_block, workspace, workspace_bytes, y_bf16, ldy, stream);
}

qd_status_t qd_int8_linear_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  qd_act_t input_act, const int8_t* w_sliced, int64_t N, const float* w_scale,
                                  const void* bias_bf16, int32_t rotate_block, void* workspace,
                                  size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream) {
    return linear_impl("qd_int8_linear_sliced", x, x_dtype, M, K, ldx, input_act, w_sliced, N, K, w_scale,
                       bias_bf16, rotate_block, workspace, workspace_bytes, y_bf16, ldy, stream, true);
}

qd_status_t qd_int8_slice_weights(const int8_t* wq, int64_t N, int64_t K, int64_t ldw, int8_t* w_sliced,
                                  hipStream_t stream) {
    const char* fn = "qd_int8_slice_weights";
    if (N < 0 || K <= 0) return fail(QD_EINVAL, fn, "need N >= 0 and K > 0 (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (K % 64 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 64", (long long)K);
    if (ldw < K) return fail(QD_EINVAL, fn, "ldw (%lld) must be >= K", (long long)ldw);
    if (N == 0) return ok();
    if (!wq || !w_sliced) return fail(QD_EINVAL, fn, "null pointer argument");
    if (!aligned16(wq) || !aligned16(w_sliced) || ldw % 16 != 0)
        return fail(QD_EUNSUPPORTED, fn, "wq, w_sliced and ldw must be 16-byte aligned");
    if (N > INT32_MAX - 256) return fail(QD_EUNSUPPORTED, fn, "N too large");
    return hip_status(fn, qd::launch_slice_weights(wq, ldw, N, K, w_sliced, stream));
}

qd_status_t qd_quantize_rowwise_act(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                    qd_act_t input_act, int32_t rotate_block, int8_t* q, int64_t ldq,
                                    float* row_scale, hipStream_t stream) {
    const char* fn = "qd_quantize_rowwise_act";
    if (rotate_block != 0 && rotate_block != 256)
        return fail(QD_EUNSUPPORTED, fn, "rotate_block must be 0 or 256 (got %d)", rotate_block);
    return quantize_impl(fn, x, x_dtype, M, K, ldx, rotate_block == 256, rotate_block, 127, q, ldq, row_scale,
                         stream, input_act);
}

qd_status_t qd_input_act(const void* x, qd_dtype_t x_dtype, int64_t n, qd_act_t act, void* out,
                         hipStream_t stream) {
    const char* fn = "qd_input_act";
    if (n < 0) return fail(QD_EINVAL, fn, "need n >= 0 (n=%lld)", (long long)n);
    if (n > 0 && (!x || !out)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (x_dtype != QD_BF16 && x_dtype != QD_F16)
        return fail(QD_EUNSUPPORTED, fn, "an input activation needs a BF16 or FP16 input");
    qd_status_t st = check_act(fn, act, x_dtype, 0);
    if (st != QD_OK) return st;
    if (((uintptr_t)x & 1u) || ((uintptr_t)out & 1u)) return fail(QD_EUNSUPPORTED, fn, "x and out must be 2-byte aligned");
    if (n == 0) return ok();
    return hip_status(fn, qd::launch_input_act(x, (int)x_dtype, n, (int)act, out, stream));
}

qd_status_t qd_dequantize_int8(const int8_t* q, int64_t M, int64_t K, int64_t ldq,
                               const float* scale, int32_t per_row, qd_dtype_t out_dtype,
                               void* out, int64_t ldo, hipStream_t stream) {
    const char* fn = "qd_dequantize_int8";
    if (M < 0 || K <= 0) return fail(QD_EINVAL, fn, "need M >= 0 and K > 0");
    if (M > 0 && (!q || !scale || !out)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (out_dtype != QD_F32 && out_dtype != QD_BF16)
        return fail(QD_EUNSUPPORTED, fn, "output dtype must be F32 or BF16");
    if (ldq < K || ldo < K) return fail(QD_EINVAL, fn, "ldq and ldo must be >= K");
    if (K % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 16", (long long)K);
    if (M > 0 && (!aligned16(q) || !aligned16(out))) return fail(QD_EUNSUPPORTED, fn, "q and out must be 16-byte aligned");
    if (ldq % 16 != 0 || (ldo * dtype_size(out_dtype)) % 16 != 0)
        return fail(QD_EUNSUPPORTED, fn, "row strides must be multiples of 16 bytes");
    if (M == 0) return ok();
    return hip_status(fn, qd::launch_dequant(q, ldq, scale, per_row != 0, out_dtype == QD_BF16, out,
                                             ldo, M, K, stream));
}

qd_status_t qd_int8_gemm_i32(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                             const int8_t* wq, int64_t N, int64_t ldw, int32_t* acc,
                             int64_t ldc, hipStream_t stream) {
    const char* fn = "qd_int8_gemm_i32";
    qd_status_t st = check_gemm(fn, aq, M, K, lda, wq, N, ldw, acc, ldc, 4);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    return hip_status(fn, qd::launch_gemm_i32(aq, lda, wq, ldw, acc, ldc, M, N, K, stream));
}

qd_status_t qd_int8_gemm_i32_sliced(const int8_t* aq, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                    const int8_t* w_sliced, int64_t N, int32_t* acc, int64_t ldc,
                                    hipStream_t stream) {
    const char* fn = "qd_int8_gemm_i32_sliced";
    if (K % 64 != 0) return fail(QD_EUNSUPPORTED, fn, "K-sliced weights need K %% 64 == 0 (K=%lld)", (long long)K);
    qd_status_t st = check_gemm(fn, aq, M, K, a_sliced ? K : lda, w_sliced, N, K, acc, ldc, 4);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    return hip_status(fn, qd::launch_gemm_i32(aq, lda, w_sliced, K, acc, ldc, M, N, K, stream, true, a_sliced != 0));
}

size_t qd_int8_attention_workspace_size(int64_t BH, int64_t Lq, int64_t Lk, int64_t D) {
    if (BH <= 0 || Lq < 0 || Lk <= 0 || D <= 0) return 0;
    const size_t rq = (size_t)BH * (size_t)Lq, rk = (size_t)BH * (size_t)Lk;
    return round_up(rq * (size_t)D, kAlign) + 2 * round_up(rk * (size_t)D, kAlign) +
           round_up(rq * sizeof(float), kAlign) + 2 * round_up(rk * sizeof(float), kAlign);
}

static qd_status_t check_attention(const char* fn, int64_t BH, int64_t Lq, int64_t Lk, int64_t D) {
    if (BH <= 0 || Lq < 0 || Lk <= 0)
        return fail(QD_EINVAL, fn, "need BH >= 1, Lq >= 0, Lk >= 1 (BH=%lld, Lq=%lld, Lk=%lld)", (long long)BH,
                    (long long)Lq, (long long)Lk);
    if (D != 64 && D != 128) return fail(QD_EUNSUPPORTED, fn, "head dim D must be 64 or 128 (got %lld)", (long long)D);
    if (BH > 65535) return fail(QD_EUNSUPPORTED, fn, "BH (%lld) exceeds 65535", (long long)BH);
    if (BH * (Lq > Lk ? Lq : Lk) > INT32_MAX) return fail(QD_EUNSUPPORTED, fn, "BH * L exceeds INT32_MAX");
    return QD_OK;
}

qd_status_t qd_int8_attention_codes(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                                    const int8_t* vc, const float* sv, int64_t BH, int64_t Lq, int64_t Lk,
                                    int64_t D, float scale, void* out_bf16, hipStream_t stream) {
    const char* fn = "qd_int8_attention_codes";
    qd_status_t st = check_attention(fn, BH, Lq, Lk, D);
    if (st != QD_OK) return st;
    if (Lq == 0) return ok();
    if (!qc || !sq || !kc || !sk || !vc || !sv || !out_bf16) return fail(QD_EINVAL, fn, "null pointer argument");
    if (((uintptr_t)qc | (uintptr_t)kc | (uintptr_t)vc | (uintptr_t)out_bf16) & 15u)
        return fail(QD_EUNSUPPORTED, fn, "codes and out must be 16-byte aligned");
    if (((uintptr_t)sq | (uintptr_t)sk | (uintptr_t)sv) & 3u)
        return fail(QD_EUNSUPPORTED, fn, "scales must be 4-byte aligned");
    const float sc = scale > 0.0f ? scale : (float)(1.0 / sqrt((double)D));
    return hip_status(fn, qd::launch_attention_i8(qc, sq, kc, sk, vc, sv, out_bf16, BH, Lq, Lk, D, sc, stream));
}

qd_status_t qd_int8_attention(const void* q, const void* k, const void* v, qd_dtype_t x_dtype, int64_t BH,
                              int64_t Lq, int64_t Lk, int64_t D, float scale, void* workspace,
                              size_t workspace_bytes, void* out_bf16, hipStream_t stream) {
    const char* fn = "qd_int8_attention";
    qd_status_t st0 = check_attention(fn, BH, Lq, Lk, D);
    if (st0 != QD_OK) return st0;
    if (!dtype_ok(x_dtype)) return fail(QD_EUNSUPPORTED, fn, "unknown input dtype %d", (int)x_dtype);
    if (Lq == 0) return ok();
    if (!q || !k || !v || !workspace || !out_bf16) return fail(QD_EINVAL, fn, "null pointer argument");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out_bf16) & 15u)
        return fail(QD_EUNSUPPORTED, fn, "q, k, v and out must be 16-byte aligned");
    if ((uintptr_t)workspace & (kAlign - 1)) return fail(QD_EUNSUPPORTED, fn, "workspace must be 256-byte aligned");
    const size_t need = qd_int8_attention_workspace_size(BH, Lq, Lk, D);
    if (workspace_bytes < need) return fail(QD_EINVAL, fn, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    const int64_t rq = BH * Lq, rk = BH * Lk;
    char* w = static_cast<char*>(workspace);
    int8_t* qc = reinterpret_cast<int8_t*>(w);
    w += round_up((size_t)rq * (size_t)D, kAlign);
    int8_t* kc = reinterpret_cast<int8_t*>(w);
    w += round_up((size_t)rk * (size_t)D, kAlign);
    int8_t* vc = reinterpret_cast<int8_t*>(w);
    w += round_up((size_t)rk * (size_t)D, kAlign);
    float* sq = reinterpret_cast<float*>(w);
    w += round_up((size_t)rq * sizeof(float), kAlign);
    float* sk = reinterpret_cast<float*>(w);
    w += round_up((size_t)rk * sizeof(float), kAlign);
    float* sv = reinterpret_cast<float*>(w);
    hipError_t e = qd::launch_rotquant(q, (int)x_dtype, false, 127, rq, D, D, qc, D, sq, stream, 0);
    if (e == hipSuccess) e = qd::launch_rotquant(k, (int)x_dtype, false, 127, rk, D, D, kc, D, sk, stream, 0);
    if (e == hipSuccess) e = qd::launch_rotquant(v, (int)x_dtype, false, 127, rk, D, D, vc, D, sv, stream, 0);
    if (e != hipSuccess) return hip_status(fn, e);
    const float sc = scale > 0.0f ? scale : (float)(1.0 / sqrt((double)D));
    return hip_status(fn, qd::launch_attention_i8(qc, sq, kc, sk, vc, sv, out_bf16, BH, Lq, Lk, D, sc, stream));
}

qd_status_t qd_set_gemm_tiles(qd_gemm_tiles_t tiles) {
    const int t = (int)tiles;
    if (t != QD_GEMM_TILES_AUTO && t != QD_GEMM_TILES_256x256 && t != QD_GEMM_TILES_256x384)
        return fail(QD_EINVAL, "qd_set_gemm_tiles", "unknown tile setting %d", t);
    static_assert((int)QD_GEMM_TILES_AUTO == qd::GEMM_TILES_AUTO && (int)QD_GEMM_TILES_256x256 == qd::GEMM_TILES_256x256 &&
                      (int)QD_GEMM_TILES_256x384 == qd::GEMM_TILES_256x384,
                  "tile settings");
    qd::set_gemm_tile_policy(t);
    return ok();
}

qd_gemm_tiles_t qd_int8_gemm_tiles(int64_t M, int64_t N, int64_t K) {
    return qd::gemm_uses_wide_tiles(M, N, K) ? QD_GEMM_TILES_256x384 : QD_GEMM_TILES_256x256;
}

qd_status_t qd_pack_int4(const int8_t* q, int64_t R, int64_t K, int64_t ldq, uint8_t* packed,
                         int64_t ldp, hipStream_t stream) {
    const char* fn = "qd_pack_int4";
    if (R < 0 || K <= 0) return fail(QD_EINVAL, fn, "need R >= 0 and K > 0");
    if (R > 0 && (!q || !packed)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (ldq < K || ldp < K / 2) return fail(QD_EINVAL, fn, "ldq must be >= K and ldp >= K/2");
    if (K % 32 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 32", (long long)K);
    if (R > 0 && (!aligned16(q) || !aligned16(packed))) return fail(QD_EUNSUPPORTED, fn, "q and packed must be 16-byte aligned");
    if (ldq % 16 != 0 || ldp % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "ldq and ldp must be multiples of 16");
    if (R == 0) return ok();
    return hip_status(fn, qd::launch_pack_int4(q, ldq, packed, ldp, R, K, stream));
}

namespace {
qd_status_t check_w4(const char* fn, int64_t K, int64_t ldw, int64_t N) {
    if (K % 64 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 64 for packed INT4 weights", (long long)K);
    if (ldw < K / 2) return fail(QD_EINVAL, fn, "ldw (%lld bytes) < K/2", (long long)ldw);
    if (ldw > QD_MAX_LD_GEMM) return fail(QD_EUNSUPPORTED, fn, "ldw (%lld) exceeds %d", (long long)ldw, QD_MAX_LD_GEMM);
    if (ldw % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "ldw must be a multiple of 16 bytes");
    (void)N;
    return QD_OK;
}
}  // namespace

qd_status_t qd_int4_scaled_mm(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                              const float* a_scale, const uint8_t* w_packed, int64_t N, int64_t ldw,
                              const float* w_scale, const void* bias_bf16, void* y_bf16,
                              int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_int4_scaled_mm";
    // validate as an INT8 GEMM with a K-byte weight stride, then the packed layout
    qd_status_t st = check_gemm(fn, aq, M, K, lda, reinterpret_cast<const int8_t*>(w_packed), N, K, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if ((st = check_w4(fn, K, ldw, N)) != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_w4_bf16(aq, lda, a_scale, w_packed, ldw, w_scale, bias_bf16, y_bf16,
                                                  ldy, M, N, K, stream));
}

qd_status_t qd_int4_gemm_i32(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                             const uint8_t* w_packed, int64_t N, int64_t ldw, int32_t* acc,
                             int64_t ldc, hipStream_t stream) {
    const char* fn = "qd_int4_gemm_i32";
    qd_status_t st = check_gemm(fn, aq, M, K, lda, reinterpret_cast<const int8_t*>(w_packed), N, K, acc, ldc, 4);
    if (st != QD_OK) return st;
    if ((st = check_w4(fn, K, ldw, N)) != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    return hip_status(fn, qd::launch_gemm_w4_i32(aq, lda, w_packed, ldw, acc, ldc, M, N, K, stream));
}

qd_status_t qd_convrot_w4a4_linear(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                   int64_t ldx, const uint8_t* w_packed, int64_t N, int64_t ldw,
                                   const float* w_scale, const void* bias_bf16,
                                   int32_t rotate_block, void* workspace, size_t workspace_bytes,
                                   void* y_bf16, int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_convrot_w4a4_linear";
    if (rotate_block != 256) return fail(QD_EUNSUPPORTED, fn, "rotate_block must be 256 (got %d)", rotate_block);
    if (M < 0 || N < 0 || K <= 0)
        return fail(QD_EINVAL, fn, "need M >= 0, N >= 0, K > 0 (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    const int64_t ldq = (int64_t)round_up((size_t)K, 16);
    if (!workspace) return fail(QD_EINVAL, fn, "null workspace");
    if ((uintptr_t)workspace % kAlign) return fail(QD_EUNSUPPORTED, fn, "workspace must be 256-byte aligned");
    if (workspace_bytes < qd_int8_linear_workspace_size(M, K))
        return fail(QD_EINVAL, fn, "workspace too small: %zu < %zu bytes", workspace_bytes,
                    qd_int8_linear_workspace_size(M, K));
    int8_t* aq = static_cast<int8_t*>(workspace);
    float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_codes_bytes(M, K));
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, true, rotate_block, aq, ldq, sx);
    if (st != QD_OK) return st;
    st = check_gemm(fn, aq, M, K, ldq, reinterpret_cast<const int8_t*>(w_packed), N, K, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if ((st = check_w4(fn, K, ldw, N)) != QD_OK) return st;
    if (!w_scale) return fail(QD_EINVAL, fn, "null w_scale");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    hipError_t e = qd::launch_rotquant(x, (int)x_dtype, true, 7, M, K, ldx, aq, ldq, sx, stream);
    if (e != hipSuccess) return hip_status(fn, e);
    return hip_status(fn, qd::launch_gemm_w4_bf16(aq, ldq, sx, w_packed, ldw, w_scale, bias_bf16, y_bf16,
                                                  ldy, M, N, K, stream));
}

// ---------------------------------------------------------------- FP6 operands

namespace {

// FP6 operand matrices: [R, K] values in 3K/4 bytes per row (the operand format
// of qdiff.h), row stride ld bytes.
qd_status_t check_f6(const char* fn, const uint8_t* a6, int64_t M, int64_t K, int64_t lda, const uint8_t* w6,
                     int64_t N, int64_t ldw, const void* out, int64_t ldo, int64_t ldo_multiple) {
    if (M < 0 || N < 0 || K <= 0)
        return fail(QD_EINVAL, fn, "need M >= 0, N >= 0, K > 0 (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N, (long long)K);
    if (M > 0 && N > 0 && (!a6 || !w6 || !out)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (K % 128 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 128 for FP6 operands", (long long)K);
    if (K > QD_MAX_K_GEMM) return fail(QD_EUNSUPPORTED, fn, "K (%lld) exceeds %d", (long long)K, QD_MAX_K_GEMM);
    if (lda < K / 4 * 3 || ldw < K / 4 * 3) return fail(QD_EINVAL, fn, "lda/ldw must be >= 3K/4 bytes");
    if (lda > QD_MAX_LD_GEMM || ldw > QD_MAX_LD_GEMM)
        return fail(QD_EUNSUPPORTED, fn, "lda/ldw (%lld, %lld) exceed %d", (long long)lda, (long long)ldw, QD_MAX_LD_GEMM);
    if (ldo < N) return fail(QD_EINVAL, fn, "output leading dimension (%lld) < N (%lld)", (long long)ldo, (long long)N);
    if (ldo > QD_MAX_LD_GEMM)
        return fail(QD_EUNSUPPORTED, fn, "output leading dimension (%lld) exceeds %d", (long long)ldo, QD_MAX_LD_GEMM);
    if (M > INT32_MAX - 256 || N > INT32_MAX - 256) return fail(QD_EUNSUPPORTED, fn, "M or N too large");
    if ((M + 255) / 256 * ((N + 255) / 256) > INT32_MAX) return fail(QD_EUNSUPPORTED, fn, "too many output tiles");
    if (M > 0 && N > 0 && (!aligned16(a6) || !aligned16(w6) || !aligned16(out)))
        return fail(QD_EUNSUPPORTED, fn, "operands and output must be 16-byte aligned");
    if (lda % 16 != 0 || ldw % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "lda and ldw must be multiples of 16 bytes");
    if (ldo % ldo_multiple != 0)
        return fail(QD_EUNSUPPORTED, fn, "output leading dimension must be a multiple of %lld", (long long)ldo_multiple);
    return QD_OK;
}

int64_t f6_ld(int64_t K) { return (int64_t)round_up((size_t)(K / 4 * 3), 16); }

}  // namespace

qd_status_t qd_pack_fp6(const int8_t* q, int64_t R, int64_t K, int64_t ldq, uint8_t* out, int64_t ldo,
                        hipStream_t stream) {
    const char* fn = "qd_pack_fp6";
    if (R < 0 || K <= 0) return fail(QD_EINVAL, fn, "need R >= 0 and K > 0 (R=%lld, K=%lld)", (long long)R, (long long)K);
    if (R > 0 && (!q || !out)) return fail(QD_EINVAL, fn, "null pointer argument");
    if (K % 64 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 64", (long long)K);
    if (ldq < K) return fail(QD_EINVAL, fn, "ldq (%lld) < K (%lld)", (long long)ldq, (long long)K);
    if (ldo < K / 4 * 3) return fail(QD_EINVAL, fn, "ldo (%lld bytes) < 3K/4", (long long)ldo);
    if (R > 0 && (!aligned16(q) || !aligned16(out))) return fail(QD_EUNSUPPORTED, fn, "q and out must be 16-byte aligned");
    if (ldq % 16 != 0 || ldo % 16 != 0) return fail(QD_EUNSUPPORTED, fn, "ldq and ldo must be multiples of 16 bytes");
    if (R == 0) return ok();
    return hip_status(fn, qd::launch_pack_fp6(q, ldq, out, ldo, R, K, stream));
}

qd_status_t qd_fp6_scaled_mm(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, const float* a_scale,
                             const uint8_t* w6, int64_t N, int64_t ldw, const float* w_scale, const void* bias_bf16,
                             void* y_bf16, int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_fp6_scaled_mm";
    qd_status_t st = check_f6(fn, a6, M, K, lda, w6, N, ldw, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_f6_bf16(a6, lda, a_scale, w6, ldw, w_scale, bias_bf16, y_bf16, ldy, M, N,
                                                  K, stream));
}

qd_status_t qd_fp6_gemm_i32(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, const uint8_t* w6, int64_t N,
                            int64_t ldw, int32_t* acc, int64_t ldc, hipStream_t stream) {
    const char* fn = "qd_fp6_gemm_i32";
    qd_status_t st = check_f6(fn, a6, M, K, lda, w6, N, ldw, acc, ldc, 4);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    return hip_status(fn, qd::launch_gemm_f6_i32(a6, lda, w6, ldw, acc, ldc, M, N, K, stream));
}

qd_status_t qd_quantize_and_rotate_rowwise_fp6(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                               int64_t ldx, int32_t block, uint8_t* q6, int64_t ld6,
                                               float* row_scale, hipStream_t stream) {
    const char* fn = "qd_quantize_and_rotate_rowwise_fp6";
    if (x_dtype != QD_BF16 && x_dtype != QD_F16)
        return fail(QD_EUNSUPPORTED, fn, "FP6 output needs a BF16 or FP16 input");
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, true, block, reinterpret_cast<int8_t*>(q6), ld6,
                                 row_scale, K / 4 * 3);
    if (st != QD_OK) return st;
    if (M == 0) return ok();
    return hip_status(fn, qd::launch_rotquant_fp6(x, (int)x_dtype, M, K, ldx, q6, ld6, row_scale, stream));
}

size_t qd_w4a4_fp6_workspace_size(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return ws_codes_bytes(M, K) + round_up((size_t)M * (size_t)f6_ld(K), kAlign) + round_up((size_t)M * sizeof(float), kAlign);
}

static qd_status_t w4a4_fp6_impl(const char* fn, const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                 int64_t ldx, const uint8_t* w6, int64_t N, int64_t ldw, const float* w_scale,
                                 const void* bias_bf16, int32_t rotate_block, void* workspace, size_t workspace_bytes,
                                 void* y_bf16, int64_t ldy, hipStream_t stream, bool sliced) {
    if (rotate_block != 256) return fail(QD_EUNSUPPORTED, fn, "rotate_block must be 256 (got %d)", rotate_block);
    if (M < 0 || N < 0 || K <= 0)
        return fail(QD_EINVAL, fn, "need M >= 0, N >= 0, K > 0 (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N, (long long)K);
    if (sliced && x_dtype != QD_BF16 && x_dtype != QD_F16)
        return fail(QD_EUNSUPPORTED, fn, "K-sliced FP6 operands need a BF16 or FP16 input");
    if (M == 0 || N == 0) return ok();
    if (!workspace) return fail(QD_EINVAL, fn, "null workspace");
    if ((uintptr_t)workspace % kAlign) return fail(QD_EUNSUPPORTED, fn, "workspace must be 256-byte aligned");
    if (workspace_bytes < qd_w4a4_fp6_workspace_size(M, K))
        return fail(QD_EINVAL, fn, "workspace too small: %zu < %zu bytes", workspace_bytes, qd_w4a4_fp6_workspace_size(M, K));
    const int64_t ldq = (int64_t)round_up((size_t)K, 16);
    const int64_t lda6 = f6_ld(K);
    char* ws = static_cast<char*>(workspace);
    int8_t* aq = reinterpret_cast<int8_t*>(ws);
    uint8_t* a6 = reinterpret_cast<uint8_t*>(ws + ws_codes_bytes(M, K));
    float* sx = reinterpret_cast<float*>(ws + ws_codes_bytes(M, K) + round_up((size_t)M * (size_t)lda6, kAlign));
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, true, rotate_block, aq, ldq, sx);
    if (st != QD_OK) return st;
    st = check_f6(fn, a6, M, K, lda6, w6, N, sliced ? K / 4 * 3 : ldw, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (!w_scale) return fail(QD_EINVAL, fn, "null w_scale");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    hipError_t e;
    if (x_dtype == QD_BF16 || x_dtype == QD_F16) {
        // 16-bit inputs: the quantizer writes the FP6 operand format itself (K-sliced for the sliced layer)
        e = qd::launch_rotquant_fp6(x, (int)x_dtype, M, K, ldx, a6, lda6, sx, stream, sliced);
    } else {
        e = qd::launch_rotquant(x, (int)x_dtype, true, 7, M, K, ldx, aq, ldq, sx, stream);
        if (e == hipSuccess) e = qd::launch_pack_fp6(aq, ldq, a6, lda6, M, K, stream);
    }
    if (e != hipSuccess) return hip_status(fn, e);
    return hip_status(fn, qd::launch_gemm_f6_bf16(a6, lda6, sx, w6, ldw, w_scale, bias_bf16, y_bf16, ldy, M, N, K,
                                                  stream, sliced, sliced));
}

qd_status_t qd_convrot_w4a4_linear_fp6(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                       const uint8_t* w6, int64_t N, int64_t ldw, const float* w_scale,
                                       const void* bias_bf16, int32_t rotate_block, void* workspace,
                                       size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream) {
    return w4a4_fp6_impl("qd_convrot_w4a4_linear_fp6", x, x_dtype, M, K, ldx, w6, N, ldw, w_scale, bias_bf16,
                         rotate_block, workspace, workspace_bytes, y_bf16, ldy, stream, false);
}

qd_status_t qd_convrot_w4a4_linear_fp6_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                              const uint8_t* w6_sliced, int64_t N, const float* w_scale,
                                              const void* bias_bf16, int32_t rotate_block, void* workspace,
                                              size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream) {
    return w4a4_fp6_impl("qd_convrot_w4a4_linear_fp6_sliced", x, x_dtype, M, K, ldx, w6_sliced, N, K / 4 * 3,
                         w_scale, bias_bf16, rotate_block, workspace, workspace_bytes, y_bf16, ldy, stream, true);
}

qd_status_t qd_fp6_slice_weights(const uint8_t* w6, int64_t N, int64_t K, int64_t ldw, uint8_t* w6_sliced,
                                 hipStream_t stream) {
    const char* fn = "qd_fp6_slice_weights";
    if (N < 0 || K <= 0) return fail(QD_EINVAL, fn, "need N >= 0 and K > 0 (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (K % 128 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 128", (long long)K);
    if (ldw < K / 4 * 3) return fail(QD_EINVAL, fn, "ldw (%lld bytes) < 3K/4", (long long)ldw);
    if (N == 0) return ok();
    if (!w6 || !w6_sliced) return fail(QD_EINVAL, fn, "null pointer argument");
    if (!aligned16(w6) || !aligned16(w6_sliced) || ldw % 16 != 0)
        return fail(QD_EUNSUPPORTED, fn, "w6, w6_sliced and ldw must be 16-byte aligned");
    if (N > INT32_MAX - 256) return fail(QD_EUNSUPPORTED, fn, "N too large");
    return hip_status(fn, qd::launch_slice_fp6(w6, ldw, N, K, w6_sliced, stream));
}

qd_status_t qd_quantize_and_rotate_rowwise_fp6_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                      int64_t ldx, int32_t block, uint8_t* q6_sliced,
                                                      float* row_scale, hipStream_t stream) {
    const char* fn = "qd_quantize_and_rotate_rowwise_fp6_sliced";
    if (x_dtype != QD_BF16 && x_dtype != QD_F16)
        return fail(QD_EUNSUPPORTED, fn, "FP6 output needs a BF16 or FP16 input");
    qd_status_t st = check_quant(fn, x, x_dtype, M, K, ldx, true, block, reinterpret_cast<int8_t*>(q6_sliced),
                                 K / 4 * 3, row_scale, K / 4 * 3);
    if (st != QD_OK) return st;
    if (K % 128 != 0) return fail(QD_EUNSUPPORTED, fn, "K (%lld) must be a multiple of 128", (long long)K);
    if (M == 0) return ok();
    return hip_status(fn, qd::launch_rotquant_fp6(x, (int)x_dtype, M, K, ldx, q6_sliced, 0, row_scale, stream, true));
}

qd_status_t qd_fp6_scaled_mm_sliced(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                    const float* a_scale, const uint8_t* w6_sliced, int64_t N, const float* w_scale,
                                    const void* bias_bf16, void* y_bf16, int64_t ldy, hipStream_t stream) {
    const char* fn = "qd_fp6_scaled_mm_sliced";
    qd_status_t st = check_f6(fn, a6, M, K, a_sliced ? K / 4 * 3 : lda, w6_sliced, N, K / 4 * 3, y_bf16, ldy, 8);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!a_scale || !w_scale) return fail(QD_EINVAL, fn, "null scale pointer");
    if (((uintptr_t)w_scale & 15u) || ((uintptr_t)bias_bf16 & 7u))
        return fail(QD_EUNSUPPORTED, fn, "w_scale must be 16-byte and bias 8-byte aligned");
    return hip_status(fn, qd::launch_gemm_f6_bf16(a6, lda, a_scale, w6_sliced, 0, w_scale, bias_bf16, y_bf16, ldy, M,
                                                  N, K, stream, true, a_sliced != 0));
}

qd_status_t qd_fp6_gemm_i32_sliced(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                   const uint8_t* w6_sliced, int64_t N, int32_t* acc, int64_t ldc,
                                   hipStream_t stream) {
    const char* fn = "qd_fp6_gemm_i32_sliced";
    qd_status_t st = check_f6(fn, a6, M, K, a_sliced ? K / 4 * 3 : lda, w6_sliced, N, K / 4 * 3, acc, ldc, 4);
    if (st != QD_OK) return st;
    if (M == 0 || N == 0) return ok();
    return hip_status(fn, qd::launch_gemm_f6_i32(a6, lda, w6_sliced, 0, acc, ldc, M, N, K, stream, true, a_sliced != 0));
}

}  // extern "C"
