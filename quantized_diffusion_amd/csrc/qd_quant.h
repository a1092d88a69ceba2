// Quantization helpers shared by the gfx950 quantizer kernels: widening of
// 16-byte input chunks, the reciprocal fast path constants, the exact code by
// the definition, and byte packing of codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qd_device.h"

namespace qd {

// Input element types: E elements per 16-byte chunk.
struct InF32 { static constexpr int E = 4; };
struct InBF16 { static constexpr int E = 8; };
struct InF16 { static constexpr int E = 8; };

// Exact widening of one 16-byte chunk to FP32.
__device__ __forceinline__ void widen(InF32, const u32x4& d, float* v) {
    v[0] = bits_f(d[0]); v[1] = bits_f(d[1]); v[2] = bits_f(d[2]); v[3] = bits_f(d[3]);
}
__device__ __forceinline__ void widen(InBF16, const u32x4& d, float* v) {
    const uint32_t w[4] = {d[0], d[1], d[2], d[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bits_f(w[i] << 16);
        v[2 * i + 1] = bits_f(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void widen(InF16, const u32x4& d, float* v) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t w[4] = {d[0], d[1], d[2], d[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h2 p = __builtin_bit_cast(h2, w[i]);
        v[2 * i] = (float)p[0];
        v[2 * i + 1] = (float)p[1];
    }
}

// Fast path: with r = fl(1/s) the code is rne(v * r) (one FMA with 1.5*2^23,
// whose low byte is the two's complement code) unless d = v*r - rne(v*r) has
// |d| >= kFastMargin; then, and for scales below kSlowScale, the element
// takes the correctly rounded division.
constexpr float kMagic = 12582912.0f;             // 1.5 * 2^23
constexpr float kFastMargin = 0.5f - 0x1p-15f;    // |d| below this: fast code is exact
constexpr float kSlowScale = 0x1p-100f;           // scales below this take the exact path

// Exact code of one element by the definition: v = fl(u * 1/16) (rotated) or
// v = u, then clamp(rne(fl(v / s))).  `w` is tau * u.  Returned as a byte.
template <bool ROT, int QMAX>
__device__ __forceinline__ uint32_t exact_code(float w, float tau, float s) {
#pragma clang fp contract(off)
    const float u = tau * w;
    const float v = ROT ? u * 0.0625f : u;
    float t = __builtin_rintf(v / s);
    t = __builtin_fminf(__builtin_fmaxf(t, (float)-QMAX), (float)QMAX);
    return (uint32_t)(int)t & 0xFFu;
}

// Low bytes of four words -> one word (a in the lowest byte).
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// FP6 E2M3 bits of four INT4 codes (bytes of w, each in [-7, 7]), one per
// byte: sign in bit 5, exponent (bias 1) in bits 4..3, mantissa in 2..0;
// every integer of [-7, 7] is exact (1 = 1.0 x 2^0 ... 7 = 1.75 x 2^2).
__device__ __forceinline__ uint32_t e2m3x4(uint32_t w) {
    const uint32_t s = (w >> 7) & 0x01010101u;        // sign per byte
    const uint32_t a = (w ^ (s * 0xFFu)) + s;          // |code| per byte (no carries: <= 7)
    const uint32_t e = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, a);   // magnitudes 0,1,2,3 | 4,5,6,7
    return e | (s << 5);
}

// Four 6-bit fields (one per byte) -> 24 bits, field i at bits 6i.
__device__ __forceinline__ uint32_t pack6x4(uint32_t c) {
    const uint32_t u = (c & 0x00FF00FFu) | (((c >> 8) & 0x00FF00FFu) << 6);
    return (u & 0xFFFu) | ((u >> 16) << 12);
}

}  // namespace qd
