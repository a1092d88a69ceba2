// Input activations folded into the quantizer's load (int8_linear's
// input_act of the comfy-kitchen 0.2.40 page, "HIP backend": an MLP's
// linear(act(proj(x))) never writes act's output to memory).
//
// The fused result equals the unfused one: act(x) rounded to nearest in the
// input's 16-bit type (BF16 or FP16, subnormals kept), then
// widened to FP32 for the rotation.  The activation is evaluated in FP64 and
// rounded once, straight onto the 16-bit grid, so the value is the correctly
// rounded activation unless the exact value lies within about 2^-50 (relative)
// of a rounding boundary; every one of the 65536 inputs of each type is
// checked against an independent evaluation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

enum { ACT_NONE = 0, ACT_GELU_TANH = 1, ACT_GELU_ERF = 2, ACT_SILU = 3, ACT_RELU = 4 };

// The activation in FP64, in forms without cancellation:
//   SiLU       x * sigmoid(x)                       = x / (1 + e^-x)
//   GELU tanh  x/2 * (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3)
//                                                   = x / (1 + e^(-2u))
//   GELU erf   x/2 * (1 + erf(x / sqrt 2))          = x/2 * erfc(-x / sqrt 2)
//   ReLU       x if x > 0, else +0
template <int ACT>
__device__ __forceinline__ double act_f64(double x) {
    if (ACT == ACT_SILU) return x / (1.0 + exp(-x));
    if (ACT == ACT_GELU_TANH) {
        const double u = 0.79788456080286535588 * (x + 0.044715 * (x * x * x));
        return x / (1.0 + exp(-2.0 * u));
    }
    if (ACT == ACT_GELU_ERF) return 0.5 * x * erfc(-x * 0.70710678118654752440);
    if (ACT == ACT_RELU) return x > 0.0 ? x : 0.0;
    return x;
}

// Round d to nearest on the grid of a binary type with MANT fraction bits and
// smallest normal exponent EMIN: spacing 2^(max(floor(log2|d|), EMIN) - MANT).
// Every step is exact in FP64 (scaling by powers of two, floor of t + 1/2 with
// |t| < 2^(MANT+1)).  An exact activation value is never halfway between grid
// points; a computed one is only when it came out as x/2 with the positive
// remainder x/2 * g(x) (g = tanh(u), tanh(x/2) or erf(x/sqrt2)) below its
// rounding error, at the smallest |x|, so halfway rounds up.
template <int MANT, int EMIN>
__device__ __forceinline__ float round_to_grid(double d) {
    if (d == 0.0) return (float)d;
    int e = ilogb(d);
    e = e < EMIN ? EMIN : e;
    double r = floor(ldexp(d, MANT - e) + 0.5);
    r = (r == 0.0 && d < 0.0) ? -0.0 : r;
    return (float)(r * ldexp(1.0, e - MANT));
}

// act(x) for an input element x (exactly widened to FP32), rounded to the
// input type IN16: 1 = BF16 (7 fraction bits, min exponent -126), 2 = FP16
// (10, -14).
template <int ACT, int IN16>
__device__ __forceinline__ float input_act(float x) {
    if (ACT == ACT_NONE) return x;
    if (ACT == ACT_RELU) return x > 0.0f ? x : 0.0f;     // exact in any type
    const double a = act_f64<ACT>((double)x);
    return IN16 == 1 ? round_to_grid<7, -126>(a) : round_to_grid<10, -14>(a);
}

// BF16 inputs of the smooth activations (GELU tanh / erf, SiLU): a BF16
// input has 65536 values, and act(x) rounded to BF16 is x itself for
// x >= 2^8, -0 for x <= -2^8, and x/2 rounded for |x| < 2^-12 (act(x) =
// x/2 + c x^2 + ..., c > 0, and the positive term is far below half an ulp,
// so only a tie moves the result: it goes up).  The 5120 inputs in between,
// 2^-12 <= |x| < 2^8, take a table built by input_act above (same values).
constexpr int kLutEmin = 115;                 // biased BF16 exponent of 2^-12
constexpr int kLutExps = 20;                  // exponents of 2^-12 .. 2^7
constexpr int kLutHalf = kLutExps * 128;      // entries per sign
constexpr int kLutN = 2 * kLutHalf;           // 5120
constexpr int kLutBytes = kLutN * 2;          // 10 KB
template <int ACT, int IN16>
struct UsesLut {
    static constexpr bool value = IN16 == 1 && (ACT == ACT_GELU_TANH || ACT == ACT_GELU_ERF || ACT == ACT_SILU);
};

// BF16 bits of the input behind table entry i (sign-major, then exponent, then mantissa).
__device__ __forceinline__ uint32_t lut_input_bits(int i) {
    const uint32_t sg = (uint32_t)(i >= kLutHalf);
    return (sg << 15) | (uint32_t)((kLutEmin << 7) + i - (int)sg * kLutHalf);
}

// act(x) as BF16 bits for BF16 bits b.
__device__ __forceinline__ uint32_t act_bf16_lut(uint32_t b, const uint16_t* lut) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const uint32_t sign = b & 0x8000u;
    if (e - (uint32_t)kLutEmin < (uint32_t)kLutExps)
        return lut[(b & 0x7FFFu) - (uint32_t)(kLutEmin << 7) + (sign >> 15) * (uint32_t)kLutHalf];
    if (e >= (uint32_t)(kLutEmin + kLutExps)) {
        if (e == 0xFFu && (b & 0x7Fu)) return b | 0x40u;    // NaN stays a (quiet) NaN
        return sign ? 0x8000u : b;                          // x (or +inf); -0 (also for -inf)
    }
    if (e >= 2u) return b - 0x80u;                          // x/2 is a normal BF16 value
    const uint32_t full = e ? (0x80u | (b & 0x7Fu)) : (b & 0x7Fu);   // |x| in units of 2^-133
    return sign | ((full >> 1) + (full & 1u & ((sign >> 15) ^ 1u)));
}

}  // namespace qd
