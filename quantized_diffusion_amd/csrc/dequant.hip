// Dequantization of INT8 codes: out[m, k] = fl(q[m, k] * s) with s per row or
// per tensor, stored as FP32 or rounded to BF16 (nearest-even).  The
// operation is dequantize_int8_simple / dequantize_int8_simple_dtype of the
// comfy-kitchen 0.2.40 page ("Huawei Ascend backend").  Memory-bound: one
// thread converts one 16-byte chunk of codes (16 outputs).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qd_device.h"
#include "qd_launch.h"
#include "qd_quant.h"

namespace qd {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                      const float* __restrict__ scale, int per_row,
                                                      uint8_t* __restrict__ out, int64_t ldo_bytes,
                                                      int64_t M, int64_t chunks_per_row) {
#pragma clang fp contract(off)
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * chunks_per_row) return;
    const int64_t m = idx / chunks_per_row;
    const int64_t c = idx - m * chunks_per_row;
    const float s = per_row ? scale[m] : scale[0];
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + m * ldq + c * 16));
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int8_t b = (int8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        v[i] = (float)b * s;
    }
    if (OUT_BF16) {
        uint8_t* dst = out + m * ldo_bytes + c * 32;
        u32x4 lo = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
        u32x4 hi = {pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                    pack_bf16x2(v[14], v[15])};
        __builtin_nontemporal_store(lo, reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(dst + 16));
    } else {
        uint8_t* dst = out + m * ldo_bytes + c * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 o = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(dst + 16 * i));
        }
    }
}

// Two signed INT4 codes per byte, code 2i in the low nibble of byte i (the
// layout convrot_w4a4_linear's packed weights use); one thread packs 32 codes.
__global__ __launch_bounds__(256) void pack_int4_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                        uint8_t* __restrict__ out, int64_t ldo, int64_t R,
                                                        int64_t chunks_per_row) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= R * chunks_per_row) return;
    const int64_t r = idx / chunks_per_row;
    const int64_t c = idx - r * chunks_per_row;
    const int8_t* src = q + r * ldq + c * 32;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + 16);
    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t t = w[i] & 0x0F0F0F0Fu;    // low nibbles of codes 4i .. 4i+3
        const uint32_t u = t | (t >> 4);          // byte 0: c0 | c1 << 4, byte 2: c2 | c3 << 4
        h[i] = (u & 0xFFu) | ((u >> 8) & 0xFF00u);
    }
    u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    *reinterpret_cast<u32x4*>(out + r * ldo + c * 16) = o;
}

// One 64-value K block of one row per thread: codes -> the FP6 operand
// format (see qdiff.h): [piece 0 bytes 0..15 | piece 1 bytes 0..15 | the
// two 8-byte tails, piece 0's first unless bits 3 and 4 of the row index differ].
__global__ __launch_bounds__(256) void pack_fp6_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                       uint8_t* __restrict__ out, int64_t ldo, int64_t R,
                                                       int64_t blocks_per_row) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= R * blocks_per_row) return;
    const int64_t r = idx / blocks_per_row;
    const int64_t b = idx - r * blocks_per_row;
    const int8_t* src = q + r * ldq + b * 64;
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + 16 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = pack6x4(e2m3x4(w[j]));
    }
    uint32_t d[12];   // the 384-bit stream of 64 fields, 24 bits per group of four
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t v0 = v[4 * g], v1 = v[4 * g + 1], v2 = v[4 * g + 2], v3 = v[4 * g + 3];
        d[3 * g] = v0 | (v1 << 24);
        d[3 * g + 1] = (v1 >> 8) | (v2 << 16);
        d[3 * g + 2] = (v2 >> 16) | (v3 << 8);
    }
    uint8_t* dst = out + r * ldo + b * 48;
    const bool swp = ((r >> 3) ^ (r >> 4)) & 1;
    *reinterpret_cast<u32x4*>(dst) = u32x4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x4*>(dst + 16) = u32x4{d[6], d[7], d[8], d[9]};
    *reinterpret_cast<u32x4*>(dst + 32) = swp ? u32x4{d[10], d[11], d[4], d[5]} : u32x4{d[4], d[5], d[10], d[11]};
}

}  // namespace

hipError_t launch_pack_fp6(const int8_t* q, int64_t ldq, uint8_t* out, int64_t ldo, int64_t R, int64_t K,
                           hipStream_t stream) {
    const int64_t bpr = K / 64;
    const int64_t grid = (R * bpr + 255) / 256;
    pack_fp6_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(q, ldq, out, ldo, R, bpr);
    return hipGetLastError();
}

hipError_t launch_pack_int4(const int8_t* q, int64_t ldq, uint8_t* out, int64_t ldo, int64_t R, int64_t K,
                            hipStream_t stream) {
    const int64_t cpr = K / 32;
    const int64_t grid = (R * cpr + 255) / 256;
    pack_int4_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(q, ldq, out, ldo, R, cpr);
    return hipGetLastError();
}

hipError_t launch_dequant(const int8_t* q, int64_t ldq, const float* scale, bool per_row,
                          bool out_bf16, void* out, int64_t ldo, int64_t M, int64_t K,
                          hipStream_t stream) {
    const int64_t cpr = K / 16;
    const int64_t total = M * cpr;
    const int64_t grid = (total + 255) / 256;
    if (out_bf16)
        dequant_kernel<true><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
            q, ldq, scale, per_row ? 1 : 0, static_cast<uint8_t*>(out), ldo * 2, M, cpr);
    else
        dequant_kernel<false><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
            q, ldq, scale, per_row ? 1 : 0, static_cast<uint8_t*>(out), ldo * 4, M, cpr);
    return hipGetLastError();
}

}  // namespace qd
