// Kernel launchers (host side).  Arguments are validated by the C ABI layer
// before these are called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

// dtype: 0 = FP32, 1 = BF16, 2 = FP16.  qmax 127 or 7 (7 only with rotate).
// act: input activation (0 none, 1 GELU tanh, 2 GELU erf, 3 SiLU, 4 ReLU);
// non-zero only with 16-bit inputs and qmax 127.
hipError_t launch_rotquant(const void* x, int dtype, bool rotate, int qmax, int64_t M, int64_t K,
                           int64_t ldx, int8_t* q, int64_t ldq, float* scale, hipStream_t stream,
                           int act = 0);

// Rotating INT4 quantizer writing the FP6 operand format directly (16-bit
// inputs, dtype 1 or 2): q6 [M, 3K/4] bytes, row stride ld6 (multiple of 16).
// The rotating INT8 quantizer writing the K-sliced code layout (byte (m, k)
// at (k / 64) * M * 64 + m * 64 + k % 64), K % 256 == 0; act as launch_rotquant.
hipError_t launch_rotquant_sliced(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                  float* scale, hipStream_t stream, int act);
// sliced: q6 in the K-sliced FP6 layout (96-byte slices, ld6 unused).
hipError_t launch_rotquant_fp6(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q6,
                               int64_t ld6, float* scale, hipStream_t stream, bool sliced = false);

// out[i] = act(x[i]) rounded to the 16-bit input type (dtype 1 BF16, 2 FP16).
hipError_t launch_input_act(const void* x, int dtype, int64_t n, int act, void* out, hipStream_t stream);

// Tensor-wise quantization: two launches; partial holds kTensorwisePartials
// floats (K % 16 == 0).
constexpr int kTensorwisePartials = 2048;
hipError_t launch_quant_tensorwise(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                   int64_t ldq, float* scale, float* partial, hipStream_t stream);
// The library's fixed partial-maxima array on the GPU that runs `stream`
// (kTensorwisePartials floats): its device address and size in floats.
hipError_t tensorwise_scratch(hipStream_t stream, float** partial, size_t* floats);

// INT8 attention on per-token codes: qc [BH*Lq, D], kc / vc [BH*Lk, D] with
// FP32 scales per row; out [BH*Lq, D] BF16; D = 64 or 128.
hipError_t launch_attention_i8(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                               const int8_t* vc, const float* sv, void* out, int64_t BH, int64_t Lq, int64_t Lk,
                               int64_t D, float scale, hipStream_t stream);

// Output tile of the INT8-weight GEMM kernels (K % 64 == 0): chosen by shape,
// or fixed (process-wide) for tuning and tests.
enum { GEMM_TILES_AUTO = 0, GEMM_TILES_256x256 = 1, GEMM_TILES_256x384 = 2 };
void set_gemm_tile_policy(int policy);
bool gemm_uses_wide_tiles(int64_t M, int64_t N, int64_t K);

// y (BF16) = epilogue(aq . wq^T); bias may be null.  a_step / w_step: 1 for a
// scale per row / per output channel, 0 for one scale for the whole operand.
// w_sliced: wq in the K-sliced layout (byte (n, k) at (k / 64) * N * 64 +
// n * 64 + k % 64, ldw unused, K % 64 == 0) instead of row-major; a_sliced:
// aq likewise (M rows, lda unused).
hipError_t launch_gemm_bf16(const int8_t* aq, int64_t lda, const float* a_scale, const int8_t* wq,
                            int64_t ldw, const float* w_scale, const void* bias, void* y,
                            int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                            int a_step = 1, int w_step = 1, bool w_sliced = false, bool a_sliced = false);

// acc (INT32) = aq . wq^T.
hipError_t launch_gemm_i32(const int8_t* aq, int64_t lda, const int8_t* wq, int64_t ldw,
                           int32_t* acc, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream, bool w_sliced = false, bool a_sliced = false);

// Row-major INT8 codes wq [N, K] (row stride ldw) -> the K-sliced layout (N * K bytes), K % 64 == 0.
hipError_t launch_slice_weights(const int8_t* wq, int64_t ldw, int64_t N, int64_t K, int8_t* out,
                                hipStream_t stream);

// Packed-INT4 weights wp [N, K/2] (row stride ldw bytes), K % 64 == 0.
hipError_t launch_gemm_w4_bf16(const int8_t* aq, int64_t lda, const float* a_scale, const uint8_t* wp,
                               int64_t ldw, const float* w_scale, const void* bias, void* y,
                               int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                               int a_step = 1, int w_step = 1);
hipError_t launch_gemm_w4_i32(const int8_t* aq, int64_t lda, const uint8_t* wp, int64_t ldw,
                              int32_t* acc, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream);

// out[r, i] = (q[r, 2i] & 15) | (q[r, 2i+1] & 15) << 4, K % 32 == 0.
hipError_t launch_pack_int4(const int8_t* q, int64_t ldq, uint8_t* out, int64_t ldo, int64_t R, int64_t K,
                            hipStream_t stream);

// INT4 codes [R, K] (K % 64 == 0) -> the FP6 E2M3 operand format, 3K/4 bytes per row.
hipError_t launch_pack_fp6(const int8_t* q, int64_t ldq, uint8_t* out, int64_t ldo, int64_t R, int64_t K,
                           hipStream_t stream);

// FP6-operand GEMM (K % 128 == 0): a6 [M, 3K/4] and w6 [N, 3K/4] bytes in the FP6
// operand format; BF16 output with the usual epilogue, or exact INT32 sums.
// w_sliced / a_sliced: that operand in the K-sliced FP6 layout (96-byte
// slices of 128 values: byte (r, b) at (b / 96) * R * 96 + r * 96 + b % 96;
// its ld unused).
hipError_t launch_gemm_f6_bf16(const uint8_t* a6, int64_t lda, const float* a_scale, const uint8_t* w6,
                               int64_t ldw, const float* w_scale, const void* bias, void* y, int64_t ldy,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream, bool w_sliced = false,
                               bool a_sliced = false);
hipError_t launch_gemm_f6_i32(const uint8_t* a6, int64_t lda, const uint8_t* w6, int64_t ldw, int32_t* acc,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                              bool w_sliced = false, bool a_sliced = false);
// Row-major FP6 operand [R, 3K/4] (row stride ld bytes) -> K-sliced (R * 3K/4 bytes), K % 128 == 0.
hipError_t launch_slice_fp6(const uint8_t* w6, int64_t ldw, int64_t N, int64_t K, uint8_t* out, hipStream_t stream);

// out = q * scale (per row or per tensor) as FP32 (out_bf16 = false) or BF16.
hipError_t launch_dequant(const int8_t* q, int64_t ldq, const float* scale, bool per_row,
                          bool out_bf16, void* out, int64_t ldo, int64_t M, int64_t K,
                          hipStream_t stream);

}  // namespace qd
