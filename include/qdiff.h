/*
 * qdiff.h -- C ABI of the MI355X (gfx950) rotated INT8 linear-layer library.
 *
 * The library computes the W8A8 "ConvRot" linear layer that the pages
 * describe: BF16 activations are rotated along K by a 256-wide block
 * Walsh-Hadamard transform, quantized per row to signed INT8 with an FP32 row
 * scale, multiplied against pre-quantized INT8 weights (per-output-channel
 * FP32 scales) with exact INT32 accumulation on the matrix cores, and the
 * result is rescaled, biased and written as BF16 in the GEMM's epilogue.
 *
 * Passages (page title, section):
 *  - comfy-kitchen 0.2.40 (PyPI), "Huawei Ascend backend": the operations
 *    quantize_int8_rowwise, quantize_and_rotate_rowwise, int8_linear,
 *    dequantize_int8_simple / _simple_dtype, convrot_w4a4_linear.
 *  - comfy-kitchen 0.2.40, "HIP backend": a K that is not a multiple of 16 is
 *    outside the kernels' domain.
 *  - SGLang PR "Tune Kitchen INT8 row splitting for SM120", "Accuracy Test":
 *    BF16 activations and bias, INT8 weights, FP32 row scales, ConvRot256.
 *  - ComfyUI-AppleSilicon-FP8 README, "What it fixes" row 17: rotate the
 *    activation online, quantize per row, INT8 x INT8 -> INT32, per-row
 *    rescale and bias fused into the store epilogue.
 *
 * Arithmetic (identical, bit for bit, to the definitions below):
 *  - rotation R: for each aligned 256-element block of a row, the
 *    Sylvester-ordered Walsh-Hadamard transform H[i][j] = (-1)^popcount(i&j)
 *    divided by 16, evaluated in FP32 as the in-place butterfly whose pair
 *    distance runs 1, 2, 4, ..., 128 (pair (j, j+h) -> (a+c, a-c)), followed
 *    by the multiply by 1/16.
 *  - row scale s = amax / qmax (one correctly rounded FP32 division), with
 *    amax = max |v| over the row and qmax = 127 (INT8) or 7 (INT4).
 *  - code = clamp(rne(fl(v / s)), -qmax, qmax); a row with s == 0 has all
 *    codes 0.
 *  - acc = sum_k a[m,k] * w[n,k] exactly in INT32.
 *  - y = bf16_rne(((float)acc * sx[m]) * sw[n] + (float)bias[n]), in FP32,
 *    left to right, no fused multiply-add.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  Matrices are
 *    row-major with a leading dimension (row stride) given in ELEMENTS.
 *  - Work is enqueued on `stream` (0 = the null stream).  No entry point
 *    allocates, frees or synchronises; results are ready when the stream
 *    reaches them.
 *  - Every argument is validated on the host before any HIP call.  On a
 *    non-QD_OK status nothing was enqueued (except QD_EHIP, which reports a
 *    failed launch), outputs are unspecified and qd_last_error() describes the
 *    problem.  Inputs are never modified.
 *  - An empty problem (M == 0, or N == 0 for the GEMMs) is valid and enqueues
 *    nothing.  K must be positive.
 *  - Calls on different streams may run concurrently as long as their output
 *    buffers (and workspaces) do not overlap.
 */
#ifndef QDIFF_H
#define QDIFF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QD_OK = 0,
    QD_EINVAL = 1,        /* null pointer, negative size, ld too small, workspace too small */
    QD_EUNSUPPORTED = 2,  /* outside the kernels' domain: K % 16, K % 256 with rotation,
                             K beyond the limit, misaligned pointer or leading dimension,
                             unknown dtype or block */
    QD_EHIP = 3           /* the HIP runtime reported an error at launch */
} qd_status_t;

typedef enum { QD_F32 = 0, QD_BF16 = 1, QD_F16 = 2 } qd_dtype_t;

/* Input activations (int8_linear's input_act, comfy-kitchen 0.2.40, "HIP
 * backend"): applied to each input element inside the quantizer's load.
 *   GELU_TANH  x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 *   GELU_ERF   x/2 (1 + erf(x / sqrt(2)))
 *   SILU       x / (1 + exp(-x))
 *   RELU       x if x > 0, else +0
 * The result is act(x) rounded to nearest-even in the input's 16-bit type
 * (what an unfused act() would store), so activations need BF16 or FP16
 * inputs. */
typedef enum { QD_ACT_NONE = 0, QD_ACT_GELU_TANH = 1, QD_ACT_GELU_ERF = 2, QD_ACT_SILU = 3,
               QD_ACT_RELU = 4 } qd_act_t;

/* Largest K accepted by the quantizers (a row stays in registers). */
#define QD_MAX_K_QUANT 65536
/* Largest K accepted by the GEMMs: the largest multiple of 16 with
 * K * 128 * 128 < 2^31, so that raw codes (including -128, accepted by the
 * GEMM entry points) can never overflow the INT32 accumulators. */
#define QD_MAX_K_GEMM 131056

/* Largest row stride the GEMMs accept, for the operands (lda, ldw: bytes of
 * INT8 codes, packed INT4 or FP6 operands) and for the output (ldy:
 * elements): a tile's copy offsets (up to 384 rows x the operand stride) and
 * its store offsets (up to 160 rows x the output stride in bytes) must fit
 * 32 bits.  Larger strides return QD_EUNSUPPORTED. */
#define QD_MAX_LD_GEMM 8388608

/* Message for the last non-OK status returned on the calling thread
 * (empty string if none).  The pointer stays valid until the next call. */
const char* qd_last_error(void);

/* Library version string. */
const char* qd_version(void);

/*
 * quantize_and_rotate_rowwise (comfy-kitchen, "Huawei Ascend backend").
 *   x          [M, K] in x_dtype (F32, BF16 or F16), row stride ldx elements.
 *   block      rotation width; must be 256.
 *   q          [M, K] INT8 codes in [-127, 127], row stride ldq bytes.
 *   row_scale  [M] FP32 scales s = amax/127 of the rotated rows.
 * Requires K % 256 == 0, K <= QD_MAX_K_QUANT, x and q 16-byte aligned,
 * ldx * sizeof(x_dtype) and ldq multiples of 16.
 * Applied to FP32 weights [N, K] this is the offline weight preparation: the
 * rotated INT8 weights and their per-output-channel scales.
 */
qd_status_t qd_quantize_and_rotate_rowwise(const void* x, qd_dtype_t x_dtype, int64_t M,
                                           int64_t K, int64_t ldx, int32_t block, int8_t* q,
                                           int64_t ldq, float* row_scale, hipStream_t stream);

/*
 * Same as qd_quantize_and_rotate_rowwise with signed INT4 codes in [-7, 7]
 * held one per byte (INT8 storage) and s = amax/7: the activation side of
 * convrot_w4a4_linear (comfy-kitchen, "Huawei Ascend backend").
 */
qd_status_t qd_quantize_and_rotate_rowwise_int4(const void* x, qd_dtype_t x_dtype, int64_t M,
                                                int64_t K, int64_t ldx, int32_t block,
                                                int8_t* q, int64_t ldq, float* row_scale,
                                                hipStream_t stream);

/*
 * quantize_int8_rowwise (comfy-kitchen, "Huawei Ascend backend"): per-row
 * dynamic symmetric INT8 quantization without rotation.  Same layout rules
 * as above except K % 16 == 0 suffices.
 */
qd_status_t qd_quantize_int8_rowwise(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                     int64_t ldx, int8_t* q, int64_t ldq, float* row_scale,
                                     hipStream_t stream);

/*
 * Quantized matmul on already quantized operands (the GEMM half of
 * int8_linear; the INT32 product never leaves the registers):
 *   y[m, n] = bf16_rne(((float)sum_k aq[m,k] * wq[n,k]) * a_scale[m] * w_scale[n] + bias[n])
 *   aq [M, K] INT8 (row stride lda bytes), a_scale [M] FP32,
 *   wq [N, K] INT8 (row stride ldw bytes), w_scale [N] FP32,
 *   bias [N] BF16 or NULL, y [M, N] BF16 (row stride ldy elements).
 * Requires K % 16 == 0, K <= QD_MAX_K_GEMM, aq/wq/y 16-byte aligned,
 * lda and ldw multiples of 16, ldy a multiple of 8, all three at most
 * QD_MAX_LD_GEMM.
 */
qd_status_t qd_int8_scaled_mm(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                              const float* a_scale, const int8_t* wq, int64_t N, int64_t ldw,
                              const float* w_scale, const void* bias_bf16, void* y_bf16,
                              int64_t ldy, hipStream_t stream);

/* Bytes of workspace qd_int8_linear needs for M rows of K: the INT8 codes
 * (rows padded to 16 bytes) and the FP32 row scales, 256-byte aligned. */
size_t qd_int8_linear_workspace_size(int64_t M, int64_t K);

/*
 * int8_linear (comfy-kitchen, "Huawei Ascend backend"; ConvRot form per the
 * SGLang PR's "Accuracy Test"): y = x W^T + b through the rotated INT8 path.
 *   x          [M, K] activations in x_dtype (BF16 on the pages), stride ldx.
 *   wq, w_scale  weights prepared offline with the SAME rotate_block
 *              (qd_quantize_and_rotate_rowwise on W [N, K]).
 *   bias       [N] BF16 or NULL.
 *   rotate_block 256 (ConvRot256) or 0 (no rotation).
 *   workspace  device buffer of at least qd_int8_linear_workspace_size(M, K)
 *              bytes, 256-byte aligned; holds the activation codes and row
 *              scales between the two launches.
 *   y          [M, N] BF16, stride ldy.
 * ldw and ldy at most QD_MAX_LD_GEMM (QD_EUNSUPPORTED above).
 * Exactly two kernels are enqueued: the (rotating) quantizer, then the INT8
 * GEMM with the fused dequantizing epilogue.
 */
qd_status_t qd_int8_linear(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                           int64_t ldx, const int8_t* wq, int64_t N, int64_t ldw,
                           const float* w_scale, const void* bias_bf16, int32_t rotate_block,
                           void* workspace, size_t workspace_bytes, void* y_bf16, int64_t ldy,
                           hipStream_t stream);

/*
 * int8_linear(input_act=...) (comfy-kitchen 0.2.40, "HIP backend": the
 * activation is folded into the quantizer's load so act's output never goes
 * to memory): y = act(x) W^T + b through the same path as qd_int8_linear,
 * where act(x) is the activation rounded to x's type.  x_dtype must be BF16
 * or FP16 when input_act != QD_ACT_NONE; with GELU or SiLU, K <= 32768.
 * Otherwise exactly qd_int8_linear (QD_ACT_NONE gives identical results).
 */
qd_status_t qd_int8_linear_act(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                               qd_act_t input_act, const int8_t* wq, int64_t N, int64_t ldw,
                               const float* w_scale, const void* bias_bf16, int32_t rotate_block,
                               void* workspace, size_t workspace_bytes, void* y_bf16, int64_t ldy,
                               hipStream_t stream);

/*
 * The quantizer half of qd_int8_linear_act: codes and row scales of act(x),
 * rotated (rotate_block 256, as qd_quantize_and_rotate_rowwise) or not
 * (rotate_block 0, as qd_quantize_int8_rowwise).  Requirements as those two
 * plus the activation's (16-bit input; K <= 32768 for GELU and SiLU).
 */
qd_status_t qd_quantize_rowwise_act(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                    qd_act_t input_act, int32_t rotate_block, int8_t* q, int64_t ldq,
                                    float* row_scale, hipStream_t stream);

/*
 * The activation alone, elementwise, by the same device code the quantizer
 * uses: out[i] = act(x[i]) in x's 16-bit type (BF16 or FP16 bits), n
 * elements, 2-byte aligned.  For verifying every input value of a type.
 */
qd_status_t qd_input_act(const void* x, qd_dtype_t x_dtype, int64_t n, qd_act_t act, void* out,
                         hipStream_t stream);

/*
 * dequantize_int8_simple / dequantize_int8_simple_dtype (comfy-kitchen,
 * "Huawei Ascend backend"): out[m, k] = fl(q[m, k] * s), s = scale[m]
 * (per_row != 0) or scale[0] (per_row == 0); out_dtype F32 or BF16 (the FP32
 * product rounded to nearest-even).
 *   q [M, K] INT8 stride ldq bytes; out [M, K] stride ldo elements.
 * Requires q and out 16-byte aligned, ldq a multiple of 16, ldo*sizeof(out)
 * a multiple of 16, K % 16 == 0.
 */
qd_status_t qd_dequantize_int8(const int8_t* q, int64_t M, int64_t K, int64_t ldq,
                               const float* scale, int32_t per_row, qd_dtype_t out_dtype,
                               void* out, int64_t ldo, hipStream_t stream);

/*
 * K-sliced INT8 weights: an offline re-layout of the weight codes that the
 * GEMM reads faster (it is an operand format of this library, not a page's).
 * Byte (n, k) of the [N, K] codes is stored at
 *     (k / 64) * N * 64 + n * 64 + k % 64,
 * i.e. the 64-byte K slices of all N rows one after another, slice by slice
 * (N * K bytes, no row stride).  Reading a weight slice then moves whole
 * 128-byte lines: one copy instruction of the GEMM fetches 1 KB of
 * consecutive bytes instead of 16 separate 64-byte pieces, which costs less
 * power per byte and lets the matrix cores run at a higher clock.  Values
 * and results are those of the row-major entry points, bit for bit.
 *
 * qd_int8_slice_weights: wq [N, K] row-major (row stride ldw bytes, a
 * multiple of 16, >= K) -> w_sliced (N * K bytes, caller-owned, 16-byte
 * aligned).  K % 64 == 0 (QD_EUNSUPPORTED otherwise).  Enqueued on stream.
 */
qd_status_t qd_int8_slice_weights(const int8_t* wq, int64_t N, int64_t K, int64_t ldw, int8_t* w_sliced,
                                  hipStream_t stream);

/*
 * qd_int8_linear_act with K-sliced weights (from qd_int8_slice_weights of
 * the codes qd_quantize_and_rotate_rowwise made, same rotate_block).  Same
 * arguments and requirements otherwise, plus K % 64 == 0; same results.
 * With rotate_block 256 the activation codes in the workspace are K-sliced
 * as well (same workspace size).
 */
qd_status_t qd_int8_linear_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  qd_act_t input_act, const int8_t* w_sliced, int64_t N, const float* w_scale,
                                  const void* bias_bf16, int32_t rotate_block, void* workspace,
                                  size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream);

/*
 * The rotating quantizer (as qd_quantize_rowwise_act with rotate_block 256;
 * QD_ACT_NONE is qd_quantize_and_rotate_rowwise) writing its codes in the
 * same K-sliced layout: byte (m, k) at (k / 64) * M * 64 + m * 64 + k % 64
 * (M * K bytes, 16-byte aligned).  qd_int8_linear_sliced keeps its
 * activation codes this way when it rotates.
 */
qd_status_t qd_quantize_and_rotate_rowwise_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                  int64_t ldx, qd_act_t input_act, int32_t block,
                                                  int8_t* q_sliced, float* row_scale, hipStream_t stream);

/*
 * qd_int8_scaled_mm with K-sliced weights (K % 64 == 0); the activation
 * codes aq are row-major with row stride lda (a_sliced == 0) or K-sliced
 * (a_sliced != 0, lda ignored).  Same results.
 */
qd_status_t qd_int8_scaled_mm_sliced(const int8_t* aq, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                     const float* a_scale, const int8_t* w_sliced, int64_t N,
                                     const float* w_scale, const void* bias_bf16, void* y_bf16,
                                     int64_t ldy, hipStream_t stream);

/* qd_int8_gemm_i32 with K-sliced weights (and aq as in qd_int8_scaled_mm_sliced); same accumulators. */
qd_status_t qd_int8_gemm_i32_sliced(const int8_t* aq, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                    const int8_t* w_sliced, int64_t N, int32_t* acc, int64_t ldc,
                                    hipStream_t stream);

/*
 * The raw INT32 accumulators of the same GEMM kernel (its INT32-store
 * epilogue), for verifying the exact contraction:
 *   acc[m, n] = sum_k aq[m, k] * wq[n, k], acc row stride ldc elements.
 * Requirements as qd_int8_scaled_mm, ldc a multiple of 4.
 */
qd_status_t qd_int8_gemm_i32(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                             const int8_t* wq, int64_t N, int64_t ldw, int32_t* acc,
                             int64_t ldc, hipStream_t stream);

/*
 * INT8 attention (int8_attention: comfy-kitchen's INT8-quantized attention
 * behind ComfyUI's --use-ck-attention, per the ai-jitan-hub article on
 * ComfyUI v0.32.0, which names the operation and says q, k and v are
 * quantized to INT8, without a formula).  This library's reading:
 *   q, k, v are quantized per token (each row of D values, per batch and
 *   head) exactly as qd_quantize_int8_rowwise does: s = amax / 127,
 *   codes clamp(rne(fl(x / s)), -127, 127);
 *   S[i][j] = (sum_d qc[i][d] * kc[j][d]) * sq[i] * sk[j] * scale (the
 *   integer sum exact, the rest FP32), softmax over j,
 *   out[i][d] = sum_j p[i][j] * sv[j] * vc[j][d] / sum_j p[i][j], BF16.
 * Layout: q [BH, Lq, D], k and v [BH, Lk, D] (BH = batch x heads), rows of
 * D contiguous, in x_dtype (QD_F32, QD_BF16 or QD_F16); out [BH, Lq, D]
 * BF16, contiguous.  scale <= 0 selects 1/sqrt(D).
 * Accuracy: the probabilities and the dequantized values sv[j] * vc[j][d]
 * enter the value product rounded to BF16 (relative error 2^-9 each), and
 * the output is rounded to BF16, so each output differs from the exact value
 * of the reading (float64 softmax of the same codes) by at most about
 * 2^-8 * max_j |sv[j] * vc[j][d]| + 2^-8 * |out| (the tests allow twice that).
 * workspace: qd_int8_attention_workspace_size(BH, Lq, Lk, D) bytes, 256-byte
 * aligned; on return it holds, in order and each part 256-byte aligned, the
 * q, k, v codes ([BH*L, D] INT8) and then their FP32 row scales.
 * Requires D == 64 or D == 128, BH >= 1, Lk >= 1 (Lq == 0 does nothing),
 * BH <= 65535, BH * max(Lq, Lk) <= 2^31 - 1, all pointers 16-byte aligned.
 * Enqueues four kernels (three quantizer launches and the attention).
 */
size_t qd_int8_attention_workspace_size(int64_t BH, int64_t Lq, int64_t Lk, int64_t D);
/* The attention step alone, on codes already quantized per token (for
 * example a cached K and V): qc [BH*Lq, D], kc / vc [BH*Lk, D] INT8, 16-byte
 * aligned; sq [BH*Lq], sk / sv [BH*Lk] FP32 row scales; out as above.
 * One kernel.  Same requirements as qd_int8_attention. */
qd_status_t qd_int8_attention_codes(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                                    const int8_t* vc, const float* sv, int64_t BH, int64_t Lq, int64_t Lk,
                                    int64_t D, float scale, void* out_bf16, hipStream_t stream);
qd_status_t qd_int8_attention(const void* q, const void* k, const void* v, qd_dtype_t x_dtype, int64_t BH,
                              int64_t Lq, int64_t Lk, int64_t D, float scale, void* workspace,
                              size_t workspace_bytes, void* out_bf16, hipStream_t stream);

/*
 * Output tile of the INT8-weight GEMM kernels (K % 64 == 0) behind
 * qd_int8_linear, qd_int8_linear_act, qd_int8_scaled_mm, qd_int8_scaled_mm_ex
 * and qd_int8_gemm_i32.  QD_GEMM_TILES_AUTO (the default) chooses 256 x 256
 * or 256 x 384 tiles by shape (the wide tile moves 17 % fewer bytes from L2
 * into LDS per MAC; the narrow one wastes less on small or ragged grids); the
 * other values fix one tile for the calling thread's later launches, for
 * tuning and for testing both kernels on the same shapes.  Results are
 * identical either way.  The setting belongs to the calling thread (each
 * thread starts with QD_GEMM_TILES_AUTO; one thread's setting never changes
 * another's launches) and is read when a GEMM is enqueued.  QD_EINVAL for
 * any other value.
 */
typedef enum { QD_GEMM_TILES_AUTO = 0, QD_GEMM_TILES_256x256 = 1, QD_GEMM_TILES_256x384 = 2 } qd_gemm_tiles_t;
qd_status_t qd_set_gemm_tiles(qd_gemm_tiles_t tiles);
/* The tile (QD_GEMM_TILES_256x256 or QD_GEMM_TILES_256x384) an INT8-weight
 * GEMM of this shape would use under the calling thread's setting. */
qd_gemm_tiles_t qd_int8_gemm_tiles(int64_t M, int64_t N, int64_t K);

/*
 * Tensor-wise scaling (comfy-kitchen 0.2.40, "Huawei Ascend backend":
 * quantize_int8_tensorwise; "HIP backend": tensor-wise is the scaling its
 * GEMMs take).
 *
 * qd_quantize_int8_tensorwise: one scale for the whole tensor, no rotation:
 *   s = amax / 127 (one correctly rounded FP32 division), amax = max |x|
 *   over all M x K elements; q[m, k] = clamp(rne(fl(x[m, k] / s)), -127, 127);
 *   s == 0 gives all-zero codes.
 *   x [M, K] in x_dtype (stride ldx elements), q [M, K] INT8 (stride ldq
 *   bytes), scale: ONE float, written.
 *   workspace: at least qd_quantize_tensorwise_workspace_size() bytes,
 *   4-byte aligned, for per-workgroup partial maxima (its contents on entry
 *   do not matter; calls that share it must not overlap).
 * Requirements as qd_quantize_int8_rowwise (K % 16 == 0, 16-byte alignment).
 * Two kernels are enqueued: partial maxima, then the quantizer.
 */
size_t qd_quantize_tensorwise_workspace_size(void);
qd_status_t qd_quantize_int8_tensorwise(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                        int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * qd_quantize_int8_tensorwise without a workspace argument.  The partial
 * maxima live in a fixed array inside the library: 2048 floats (8 KB), one
 * copy per GPU, held until the process ends.  The partial count is
 * min(M, 2048), so every input qd_quantize_int8_tensorwise accepts fits;
 * a count above the array would be QD_EUNSUPPORTED.  Arguments, results
 * (bit for bit) and errors as qd_quantize_int8_tensorwise; QD_EHIP if the
 * array's device address cannot be found.  Allocates and frees nothing.
 * Every call on one GPU uses the same array, and each call writes every
 * partial it reads before reading it (nothing needs clearing), so calls in
 * one stream order are safe; calls that overlap on one GPU (other streams
 * or threads) race and must be serialised by the caller.
 */
qd_status_t qd_quantize_int8_tensorwise_noalloc(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                                hipStream_t stream);

/*
 * qd_int8_scaled_mm with the scale granularity chosen per operand:
 *   y[m, n] = bf16_rne(((float)acc[m, n] * sa(m)) * sw(n) + bias[n]),
 *   sa(m) = a_scale[m] if a_scale_len == M, a_scale[0] if a_scale_len == 1;
 *   sw(n) = w_scale[n] if w_scale_len == N, w_scale[0] if w_scale_len == 1.
 * (1, 1) is the tensor-wise GEMM; (M, N) is qd_int8_scaled_mm.  Other
 * lengths are QD_EINVAL.  A per-channel w_scale must be 16-byte aligned.
 * Otherwise as qd_int8_scaled_mm.
 */
qd_status_t qd_int8_scaled_mm_ex(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                                 const float* a_scale, int64_t a_scale_len, const int8_t* wq,
                                 int64_t N, int64_t ldw, const float* w_scale, int64_t w_scale_len,
                                 const void* bias_bf16, void* y_bf16, int64_t ldy, hipStream_t stream);

/*
 * INT4 storage for convrot_w4a4_linear (comfy-kitchen 0.2.40, "Huawei Ascend
 * backend": signed INT4 activation codes kept in INT8 storage, packed INT4
 * weights unpacked to INT8 for INT32 accumulation).
 *
 * qd_pack_int4: packed[r, i] = (q[r, 2i] & 15) | (q[r, 2i+1] & 15) << 4 for
 * codes in [-8, 7] (two's complement nibbles, code 2i in the low nibble).
 *   q [R, K] INT8 (row stride ldq bytes), packed [R, K/2] (row stride ldp
 *   bytes).  Requires K % 32 == 0, q/packed 16-byte aligned, ldq and ldp
 *   multiples of 16, ldp >= K/2.
 */
qd_status_t qd_pack_int4(const int8_t* q, int64_t R, int64_t K, int64_t ldq, uint8_t* packed,
                         int64_t ldp, hipStream_t stream);

/*
 * The GEMM half of convrot_w4a4_linear: as qd_int8_scaled_mm with the weights
 * given as packed INT4 w_packed [N, K/2] (row stride ldw BYTES), unpacked to
 * INT8 inside the kernel.  Requires K % 64 == 0, ldw a multiple of 16 and
 * >= K/2, otherwise as qd_int8_scaled_mm.
 */
qd_status_t qd_int4_scaled_mm(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                              const float* a_scale, const uint8_t* w_packed, int64_t N, int64_t ldw,
                              const float* w_scale, const void* bias_bf16, void* y_bf16,
                              int64_t ldy, hipStream_t stream);

/* Raw INT32 accumulators of the packed-INT4 GEMM (verification). */
qd_status_t qd_int4_gemm_i32(const int8_t* aq, int64_t M, int64_t K, int64_t lda,
                             const uint8_t* w_packed, int64_t N, int64_t ldw, int32_t* acc,
                             int64_t ldc, hipStream_t stream);

/*
 * convrot_w4a4_linear: y = x W^T + b through the rotated INT4 path.  x is
 * rotated (block 256) and quantized per row to INT4 codes in INT8 storage
 * (s = amax / 7); w_packed [N, K/2] / w_scale [N] come from
 * qd_quantize_and_rotate_rowwise_int4 on W followed by qd_pack_int4.
 * rotate_block must be 256; K % 256 == 0.  Workspace as qd_int8_linear
 * (qd_int8_linear_workspace_size).  Two kernels: quantizer, then GEMM.
 */
qd_status_t qd_convrot_w4a4_linear(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                   int64_t ldx, const uint8_t* w_packed, int64_t N, int64_t ldw,
                                   const float* w_scale, const void* bias_bf16,
                                   int32_t rotate_block, void* workspace, size_t workspace_bytes,
                                   void* y_bf16, int64_t ldy, hipStream_t stream);

/*
 * W4A4 on the FP6 matrix path (the "map INT4 codes to FP6 E2M3" option for
 * convrot_w4a4_linear).  Every INT4 code in [-7, 7] is exact in FP6 E2M3
 * (OCP MX: sign, 2 exponent bits with bias 1, 3 mantissa bits), and all
 * partial sums are integers below K * 49 < 2^24, so the FP32 accumulation
 * of gfx950's FP6 matrix instructions is exact and the results equal the
 * INT8-path results bit for bit.
 *
 * FP6 operand format of an [R, K] matrix (K % 64 == 0): each row takes 3K/4
 * bytes (row stride ld bytes, a multiple of 16).  Values 64j .. 64j+63 of a
 * row fill the 48 bytes at 48j as two pieces of 32 values (piece p = values
 * 64j + 32p .. +31, value i of a piece in bits 6i .. 6i+5 of its 24 bytes,
 * least significant first):
 *     bytes  0..15  piece 0 bytes 0..15
 *     bytes 16..31  piece 1 bytes 0..15
 *     bytes 32..47  piece 0 bytes 16..23 then piece 1 bytes 16..23, or the
 *                   two swapped when bits 3 and 4 of the row index differ.
 *
 * qd_pack_fp6: codes q [R, K] INT8 in [-7, 7] (other values give undefined
 * bytes) -> out [R, 3K/4] in that format.  K % 64 == 0; q/out 16-byte
 * aligned; ldq, ldo multiples of 16; ldo >= 3K/4.
 */
qd_status_t qd_pack_fp6(const int8_t* q, int64_t R, int64_t K, int64_t ldq, uint8_t* out, int64_t ldo,
                        hipStream_t stream);

/*
 * The rotating INT4 quantizer (as qd_quantize_and_rotate_rowwise_int4) writing
 * the codes straight into the FP6 operand format: q6 [M, 3K/4] bytes, row
 * stride ld6 bytes (>= 3K/4, a multiple of 16), row_scale [M].  BF16 or FP16
 * input; block 256, K % 256 == 0.
 */
qd_status_t qd_quantize_and_rotate_rowwise_fp6(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                               int64_t ldx, int32_t block, uint8_t* q6, int64_t ld6,
                                               float* row_scale, hipStream_t stream);

/*
 * The GEMM on FP6 operands: a6 [M, 3K/4] (stride lda bytes) and w6
 * [N, 3K/4] (stride ldw bytes) in the FP6 operand format, a_scale [M],
 * w_scale [N], bias [N] BF16 or NULL, y [M, N] BF16:
 *   y = bf16_rne(((float)sum_k a[m,k] w[n,k] * a_scale[m]) * w_scale[n] + bias[n]).
 * K % 128 == 0, K <= QD_MAX_K_GEMM; otherwise as qd_int8_scaled_mm.
 * qd_fp6_gemm_i32 writes the exact sums as INT32 (ldc a multiple of 4).
 */
qd_status_t qd_fp6_scaled_mm(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, const float* a_scale,
                             const uint8_t* w6, int64_t N, int64_t ldw, const float* w_scale, const void* bias_bf16,
                             void* y_bf16, int64_t ldy, hipStream_t stream);
qd_status_t qd_fp6_gemm_i32(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, const uint8_t* w6, int64_t N,
                            int64_t ldw, int32_t* acc, int64_t ldc, hipStream_t stream);

/*
 * convrot_w4a4_linear with FP6 weights w6 [N, 3K/4] (qd_quantize_and_rotate_rowwise_int4
 * on W, then qd_pack_fp6): the rotating INT4 quantizer writing FP6 (BF16 or
 * FP16 x; FP32 x: INT4 codes, then qd_pack_fp6), then the FP6 GEMM.  Same
 * results as qd_convrot_w4a4_linear.
 * K % 256 == 0; workspace of qd_w4a4_fp6_workspace_size(M, K) bytes,
 * 256-byte aligned.
 */
size_t qd_w4a4_fp6_workspace_size(int64_t M, int64_t K);
qd_status_t qd_convrot_w4a4_linear_fp6(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                       const uint8_t* w6, int64_t N, int64_t ldw, const float* w_scale,
                                       const void* bias_bf16, int32_t rotate_block, void* workspace,
                                       size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream);

/*
 * K-sliced FP6 operands (the FP6 counterpart of the K-sliced INT8 layout
 * above): byte b of row r of an FP6 operand ([R, 3K/4] bytes, K % 128 == 0)
 * stored at (b / 96) * R * 96 + r * 96 + b % 96, i.e. the 96-byte slices
 * of 128 values of all rows one after another (R * 3K/4 bytes).  Row-major
 * FP6 rows are 96 bytes per slice and straddle 128-byte lines; K-sliced,
 * a copy instruction of the GEMM reads 1 KB of consecutive bytes.  Same
 * values, same results as the row-major entry points, bit for bit.
 *
 * qd_fp6_slice_weights: w6 [N, 3K/4] row-major (row stride ldw bytes, a
 * multiple of 16) -> w6_sliced (caller-owned, 16-byte aligned).
 * qd_quantize_and_rotate_rowwise_fp6_sliced: as qd_quantize_and_rotate_rowwise_fp6
 * with the K-sliced output (BF16 or FP16 input, K % 256 == 0).
 * qd_fp6_scaled_mm_sliced / qd_fp6_gemm_i32_sliced: as qd_fp6_scaled_mm /
 * qd_fp6_gemm_i32 with K-sliced weights; a6 row-major with row stride lda
 * (a_sliced == 0) or K-sliced (a_sliced != 0, lda ignored).
 * qd_convrot_w4a4_linear_fp6_sliced: the layer with K-sliced weights, its
 * quantizer writing the activation operand K-sliced into the workspace
 * (same size as qd_w4a4_fp6_workspace_size); BF16 or FP16 input only.
 */
qd_status_t qd_fp6_slice_weights(const uint8_t* w6, int64_t N, int64_t K, int64_t ldw, uint8_t* w6_sliced,
                                 hipStream_t stream);
qd_status_t qd_quantize_and_rotate_rowwise_fp6_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K,
                                                      int64_t ldx, int32_t block, uint8_t* q6_sliced,
                                                      float* row_scale, hipStream_t stream);
qd_status_t qd_fp6_scaled_mm_sliced(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                    const float* a_scale, const uint8_t* w6_sliced, int64_t N, const float* w_scale,
                                    const void* bias_bf16, void* y_bf16, int64_t ldy, hipStream_t stream);
qd_status_t qd_fp6_gemm_i32_sliced(const uint8_t* a6, int64_t M, int64_t K, int64_t lda, int32_t a_sliced,
                                   const uint8_t* w6_sliced, int64_t N, int32_t* acc, int64_t ldc,
                                   hipStream_t stream);
qd_status_t qd_convrot_w4a4_linear_fp6_sliced(const void* x, qd_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                              const uint8_t* w6_sliced, int64_t N, const float* w_scale,
                                              const void* bias_bf16, int32_t rotate_block, void* workspace,
                                              size_t workspace_bytes, void* y_bf16, int64_t ldy, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QDIFF_H */
