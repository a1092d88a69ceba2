// Rotate-and-quantize kernel for gfx950 (CDNA4).
//
// Computes, per row of x, the block-256 normalised Walsh-Hadamard rotation
// (Sylvester order, FP32 butterfly with pair distance 1, 2, ..., 128, then
// x 1/16), the row scale s = amax / qmax and the codes
// clamp(rne(fl(v / s)), -qmax, qmax).  The operation is the one the
// comfy-kitchen 0.2.40 page lists as quantize_and_rotate_rowwise ("Huawei
// Ascend backend"); the rotation is the ConvRot256 of the SGLang PR
// "Tune Kitchen INT8 row splitting for SM120" ("Accuracy Test").  With
// ROT == false the same kernel is quantize_int8_rowwise.
//
// Work layout.  Four lanes (a "quad") own one 256-element block: lane ql of
// the quad holds the 16-byte chunks c = 4*i + ql (i = 0 .. NI-1) of the
// block, so each load instruction of a quad reads 64 contiguous bytes and a
// wave reads 16 such pieces of consecutive blocks.  With E elements per
// chunk the element index is (4*i + ql)*E + e, so butterfly stages on the
// bits of e and of i stay inside a lane's registers and the two stages on
// the bits of ql cross lanes through DPP quad permutes.
//
// Cross-lane stages without per-lane opcodes: a lane computes
// own + c * partner with c = +1 in the lower lane of the pair and -1 in the
// upper lane.  The lower lane gets a + c exactly as the butterfly does; the
// upper lane gets c - a, the exact negation of a - c (round-to-nearest is
// symmetric).  Both lanes of every later pair carry the same sign, so each
// lane's values are the true values times tau = (-1)^popcount(ql), and the
// sign is folded into the reciprocal of the scale when quantizing.
//
// Quantization without a division per element.  With r = fl(1/s) the exact
// product x = v*r differs from Q = v/s by at most |Q|*2^-24 < 2^-17, and
// |fl(Q) - Q| <= 2^-18 for |Q| < 128.  The code is taken as rne(x) (one FMA
// with 1.5*2^23); a second FMA gives d = x - rne(x).  When |d| < 0.5 - 2^-15,
// fl(Q) lies strictly within 0.5 of the same integer, so rne(fl(Q)) equals
// it.  Otherwise (about 6e-5 of the elements) the element is redone with the
// correctly rounded division, which is also used for whole rows whose scale
// is below 2^-100.  The 1/16 of the rotation is applied to amax and to r
// (powers of two, exact); the slow path applies it to the element exactly as
// the definition does.
//
// Row amax: per-lane max, quad reduction by DPP, then an LDS atomic max over
// the blocks of the row (non-negative floats order like their bit patterns).
//
// Memory: a quad's load instruction covers half a 128-byte line and the next
// one the other half, so loads use the default cache policy (the L2 merges
// the halves; streaming hints would fetch partial lines).  The codes of the
// rotated path are staged through LDS per wave: each lane writes its chunks
// into its quad's 256-byte block image, then lane l stores bytes
// [16 l, 16 l + 16) of four consecutive block images, so one store
// instruction writes four whole blocks (1 KB, whole 128-byte lines).  The
// stores keep the default cache policy: the GEMM reads the codes next, and a
// whole step measured faster that way than with streaming stores.
//
// K-sliced output (SL, for the GEMM's K-sliced operand layout): byte (m, k)
// goes to (k / S) * M * S + m * S + k % S with S = 64 for INT8 codes and
// S = 96 bytes (128 values) for the FP6 operand; a block image leaves LDS as
// its 64- or 96-byte slice pieces.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qd_device.h"
#include "qd_launch.h"
#include "qd_quant.h"
#include "qd_act.h"

namespace qd {

typedef float f32x16 __attribute__((ext_vector_type(16)));
namespace {

template <class In> struct In16 { static constexpr int value = 0; };
template <> struct In16<InBF16> { static constexpr int value = 1; };
template <> struct In16<InF16> { static constexpr int value = 2; };

// act() on the eight 16-bit values of a chunk, results in the same type
// (BF16 with a smooth activation: the table lut; otherwise FP64 evaluation).
template <int ACT, int IN16>
__device__ __forceinline__ u32x4 act_chunk(u32x4 d, const uint16_t* lut) {
    if (IN16 == 0) return d;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t out = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t b = (d[w] >> (16 * h)) & 0xFFFFu;
            uint32_t r;
            if (UsesLut<ACT, IN16>::value) {
                r = act_bf16_lut(b, lut);   // chunks with an input outside the table
            } else {
                const float f = IN16 == 1 ? bits_f(b << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)b);
                const float a = input_act<ACT, IN16>(f);
                r = IN16 == 1 ? f_bits(a) >> 16 : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a);
            }
            out |= r << (16 * h);
        }
        d[w] = out;
    }
    return d;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// act() on a BF16 chunk through the table: indices two at a time in 16-bit
// lanes (entry = |x| bits - 2^-12's bits, + kLutHalf for negative x), one
// range test for the chunk, the general path only for a chunk with an input
// outside the table.
template <int ACT>
__device__ __forceinline__ u32x4 act_chunk_lut(u32x4 d, const uint16_t* lut) {
    u16x2 t[4], idx[4];
    const u16x2 base = {(unsigned short)(kLutEmin << 7), (unsigned short)(kLutEmin << 7)};
    const u16x2 half = {(unsigned short)kLutHalf, (unsigned short)kLutHalf};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        t[w] = __builtin_bit_cast(u16x2, d[w] & 0x7FFF7FFFu) - base;
        const u16x2 sg = __builtin_bit_cast(u16x2, (d[w] >> 15) & 0x00010001u);
        idx[w] = sg * half + t[w];
    }
    const u16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(t[0], t[1]),
                                               __builtin_elementwise_max(t[2], t[3]));
    if (__builtin_expect(mx[0] < (unsigned short)kLutHalf && mx[1] < (unsigned short)kLutHalf, 1)) {
#pragma unroll
        for (int w = 0; w < 4; ++w) d[w] = (uint32_t)lut[idx[w][0]] | ((uint32_t)lut[idx[w][1]] << 16);
        return d;
    }
    return act_chunk<ACT, 1>(d, lut);
}

// Tables of the smooth activations for BF16 inputs (entry i: input
// lut_input_bits(i)), rebuilt by act_lut_kernel on the stream of every
// launch that reads them.  The values never change, so launches on other
// streams that rebuild a table concurrently only rewrite the same bits.
__device__ uint16_t g_act_lut[3][kLutN];

template <int ACT>
__global__ __launch_bounds__(256) void act_lut_kernel() {
    const int i = blockIdx.x * 256 + (int)threadIdx.x;
    if (i < kLutN) {
        const float x = bits_f(lut_input_bits(i) << 16);
        g_act_lut[ACT - 1][i] = (uint16_t)(f_bits(input_act<ACT, 1>(x)) >> 16);
    }
}

template <int ACT, int IN16>
hipError_t build_lut(hipStream_t stream) {
    if (!UsesLut<ACT, IN16>::value) return hipSuccess;
    act_lut_kernel<UsesLut<ACT, IN16>::value ? ACT : ACT_SILU><<<dim3((kLutN + 255) / 256), dim3(256), 0, stream>>>();
    return hipGetLastError();
}

// Largest workgroup: 1024 threads (4 waves per SIMD, 128 VGPRs); 512 with an
// FP64 activation, whose temporaries need more registers.
template <int ACT, int IN16>
struct kMaxThreads {
    static constexpr int value = (ACT == 0 || ACT == 4 || UsesLut<ACT, IN16>::value) ? 1024 : 512;
};

constexpr int kStageStride = 288;                 // bytes per block image in LDS (256 + 32: spreads banks)
constexpr int kStageWave = 16 * kStageStride;     // per wave: 16 quads
// Whole-line code stores.  The codes are read again by the GEMM that follows
// (and fit the Infinity Cache at the sizes used), so they are stored with the
// default policy unless kStreamCodes is set.
constexpr bool kStreamCodes = false;
__device__ __forceinline__ void store_codes(const u32x4& v, int8_t* dst) {
    if (kStreamCodes) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
    else *reinterpret_cast<u32x4*>(dst) = v;
}
constexpr int kF6Stride = 208;                    // FP6 block image: 192 bytes (+16: an odd count of 16-byte slots)
constexpr int kF6Wave = 16 * kF6Stride;

// One cross-lane butterfly stage for one value: own + sign * partner, the
// partner read through DPP inside the FMA (a separate v_mov_b32_dpp would
// double the VALU work of the stage).  The two wait states cover the
// hazard of a DPP read of a VGPR written by the previous VALU instruction.
__device__ __forceinline__ float fmac_quad_xor1(float own, float sign) {
    asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                 : "+v"(own) : "v"(sign));
    return own;
}
__device__ __forceinline__ float fmac_quad_xor2(float own, float sign) {
    asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                 : "+v"(own) : "v"(sign));
    return own;
}

template <class In, bool ROT, int QMAX, bool STAGE, bool F6>
__device__ __forceinline__ void quantize_store(const float* v, uint32_t amax_bits, int row, int blk,
                                               int ql, int K, int8_t* __restrict__ q, int64_t ldq,
                                               float* __restrict__ scale, uint8_t* img);

// STAGE (rotated path only): codes leave through the LDS block images.
// ACT: input activation applied to each widened element (16-bit inputs).
// F6 (INT4 codes, 16-bit inputs, STAGE): the codes are written as FP6 E2M3
// fields straight into the FP6 operand format (q is then the FP6 matrix,
// ldq its row stride in bytes, 3K/4 bytes per row): each 8-code chunk is
// 48 bits, three 2-byte pieces placed in the block's 192-byte image at their
// head / tail positions.  The fields of four chunks come from one gfx950
// FP32 -> FP6 conversion (v_cvt_scalef32_2xpk16_fp6_f32, unit scale) of the
// codes as floats, which are exact integers of [-7, 7].
template <class In, bool ROT, int QMAX, bool STAGE, int ACT, bool F6 = false, bool SL = false>
__global__ __launch_bounds__((kMaxThreads<ACT, In16<In>::value>::value)) void rotquant_kernel(const uint8_t* __restrict__ x,
                                                        int64_t ldx_bytes, int M, int K, int nb,
                                                        int R, int8_t* __restrict__ q,
                                                        int64_t ldq, float* __restrict__ scale) {
    constexpr int E = In::E;             // elements per 16-byte chunk
    constexpr int NI = 256 / (4 * E);    // chunks per lane per block
    constexpr int NV = NI * E;           // 64 values per lane
    constexpr int ESZ = 16 / E;          // bytes per input element
    __shared__ uint32_t row_amax[256];
    // dynamic LDS: [activation table (LUT) | kStageWave per wave (rotated path)]
    constexpr bool LUT = UsesLut<ACT, In16<In>::value>::value;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    uint8_t* const stage = lds_dyn + (LUT ? kLutBytes : 0);
    const uint16_t* lut = reinterpret_cast<const uint16_t*>(lds_dyn);
    auto load_lut = [&]() {
        if (LUT) {
            const u32x4* src = reinterpret_cast<const u32x4*>(g_act_lut[(ACT > 0 && ACT < 4) ? ACT - 1 : 0]);
            for (int c = threadIdx.x; c < kLutBytes / 16; c += blockDim.x)
                reinterpret_cast<u32x4*>(lds_dyn)[c] = src[c];
            __syncthreads();
        }
    };

    const int tid = threadIdx.x;
    const int quad = tid >> 2;
    const int ql = tid & 3;
    // quad / nb by a 24-bit multiply: with inv = ceil(2^20 / nb) the error of
    // quad * inv / 2^20 is below quad / 2^20 < 1/nb for quad < 4096.
    const uint32_t nb_inv = ((1u << 20) + nb - 1) / nb;
    const int rl = (int)(__umul24((uint32_t)quad, nb_inv) >> 20);
    const int blk = quad - rl * nb;
    // K-sliced output (SL): the row groups of one XCD (workgroups g with the
    // same g % 8) are consecutive, so the neighbouring rows whose codes share
    // a 128-byte line of a slice are written through the same L2
    const int G = (int)gridDim.x, g = (int)blockIdx.x;
    const int wg = SL ? (g % 8) * (G / 8) + min(g % 8, G % 8) + g / 8 : g;
    const int row = wg * R + rl;
    const bool active = (rl < R) && (row < M);
    if (tid < R) row_amax[tid] = 0u;

    float v[NV];
    if (ROT) {
        // Whole blocks: every lane loads (idle quads read a valid row and
        // discard the result), so the loads need neither a branch nor zeroed
        // registers.  Quads never mix active and idle lanes.
        const int lrow = min(min(wg * R + min(rl, R - 1), row), M - 1);
        const uint8_t* src = x + (int64_t)lrow * ldx_bytes + (int64_t)blk * 256 * ESZ;
        u32x4 d[NI];
        // The sliced INT8 quantizer feeds the wide GEMM: x is read once, so a
        // non-temporal load keeps it from displacing the GEMM's operands in L2
        // and the memory-side cache.
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const u32x4* p = reinterpret_cast<const u32x4*>(src + (i * 4 + ql) * 16);
            d[i] = (SL && !F6) ? __builtin_nontemporal_load(p) : *p;
        }
        if (ACT != ACT_NONE) {
            load_lut();
            // on the raw 16-bit words, before widening: fewer live registers
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                d[i] = LUT ? act_chunk_lut<ACT>(d[i], lut) : act_chunk<ACT, In16<In>::value>(d[i], lut);
                __builtin_amdgcn_sched_barrier(0);   // one chunk at a time: bounded FP64 temporaries
            }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) widen(In{}, d[i], &v[i * E]);
    } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = 0.0f;
        if (ACT != ACT_NONE) load_lut();
        if (active) {
            const uint8_t* src = x + (int64_t)row * ldx_bytes + (int64_t)blk * 256 * ESZ;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int c = i * 4 + ql;
                if (blk * 256 + c * E < K) {
                    u32x4 d = *reinterpret_cast<const u32x4*>(src + c * 16);
                    if (ACT != ACT_NONE)
                        d = LUT ? act_chunk_lut<ACT>(d, lut) : act_chunk<ACT, In16<In>::value>(d, lut);
                    widen(In{}, d, &v[i * E]);
                }
            }
        }
    }

    if (ROT) {
        // stages on the element bits inside a chunk
#pragma unroll
        for (int h = 1; h < E; h *= 2) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                if (!(j & h)) {
                    const float a = v[j], c = v[j + h];
                    v[j] = a + c;
                    v[j + h] = a - c;
                }
            }
        }
        // stages on the two quad-lane bits (pair distance E and 2E)
        const float c0 = (ql & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = fmac_quad_xor1(v[j], c0);
        const float c1 = (ql & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = fmac_quad_xor2(v[j], c1);
        // stages on the chunk-index bits (pair distance 4E, 8E, ...)
#pragma unroll
        for (int hi = 1; hi < NI; hi *= 2) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (!(i & hi)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float a = v[i * E + e], c = v[(i + hi) * E + e];
                        v[i * E + e] = a + c;
                        v[(i + hi) * E + e] = a - c;
                    }
                }
            }
        }
    }

    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(v[j]));
    am = __builtin_fmaxf(am, quad_xor1(am));
    am = __builtin_fmaxf(am, quad_xor2(am));
    __syncthreads();
    if (active && ql == 0) atomicMax(&row_amax[rl], f_bits(am));
    __syncthreads();
    if (active) {
        uint8_t* img = F6 ? stage + (tid >> 6) * kF6Wave + ((tid >> 2) & 15) * kF6Stride
                          : stage + (tid >> 6) * kStageWave + ((tid >> 2) & 15) * kStageStride;
        quantize_store<In, ROT, QMAX, STAGE, F6>(v, row_amax[rl], row, blk, ql, K, q, ldq, scale, img);
    }
    if (F6) {
        // twelve 16-byte slots per block image; lane l stores slots l, l+64, l+128 of the wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int lane = tid & 63;
        const uint8_t* imgs = stage + (tid >> 6) * kF6Wave;
        u32x4 val[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int sl = lane + 64 * j;
            val[j] = *reinterpret_cast<const u32x4*>(imgs + (sl / 12) * kF6Stride + 16 * (sl % 12));
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int sl = lane + 64 * j;
            const int qq = (tid >> 6) * 16 + sl / 12;
            const int rl2 = (int)(__umul24((uint32_t)qq, nb_inv) >> 20);
            const int row2 = wg * R + rl2;
            if (rl2 < R && row2 < M) {
                // SL: K-sliced FP6 operand, 96-byte slices, ldq = the slice stride (M * 96 bytes)
                const int blk2 = qq - rl2 * nb, kb = 16 * (sl % 12);
                int8_t* dst = SL ? q + (int64_t)(2 * blk2 + kb / 96) * ldq + (int64_t)row2 * 96 + kb % 96
                                 : q + (int64_t)row2 * ldq + blk2 * 192 + kb;
                store_codes(val[j], dst);
            }
        }
    } else if (STAGE) {
        // Whole-block stores of the wave's 16 block images (see the header).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int lane = tid & 63;
        const uint8_t* img = stage + (tid >> 6) * kStageWave + (lane >> 4) * kStageStride + 16 * (lane & 15);
        u32x4 val[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) val[j] = *reinterpret_cast<const u32x4*>(img + 4 * j * kStageStride);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qq = (tid >> 6) * 16 + 4 * j + (lane >> 4);   // quad of the workgroup
            const int rl2 = (int)(__umul24((uint32_t)qq, nb_inv) >> 20);
            const int row2 = wg * R + rl2;
            if (rl2 < R && row2 < M) {
                // SL: K-sliced codes, ldq = the slice stride (M * 64 bytes)
                const int blk2 = qq - rl2 * nb, kin = 16 * (lane & 15);
                int8_t* dst = SL ? q + (int64_t)(4 * blk2 + (kin >> 6)) * ldq + (int64_t)row2 * 64 + (kin & 63)
                                 : q + (int64_t)row2 * ldq + blk2 * 256 + kin;
                store_codes(val[j], dst);
            }
        }
    }
}

// Scale and codes of one quad's values (see the header).  Rotated path: the
// codes go to the quad's block image `img` in LDS; otherwise straight to q.
template <class In, bool ROT, int QMAX, bool STAGE, bool F6>
__device__ __forceinline__ void quantize_store(const float* v, uint32_t amax_bits, int row, int blk,
                                               int ql, int K, int8_t* __restrict__ q, int64_t ldq,
                                               float* __restrict__ scale, uint8_t* img) {
    constexpr int E = In::E;
    constexpr int NI = 256 / (4 * E);
    const float amax_u = bits_f(amax_bits);
    const float amax = ROT ? amax_u * 0.0625f : amax_u;
    const float s = amax / (float)QMAX;
    if (blk == 0 && ql == 0) scale[row] = s;
    const float tau = (ROT && ((ql ^ (ql >> 1)) & 1)) ? -1.0f : 1.0f;

    // Per row: 0 = all codes zero, 1 = fast path with exact fallback,
    // 2 = exact division for every element (tiny scales).
    const int mode = (s >= kSlowScale) ? 1 : (s == 0.0f ? 0 : 2);
    const float r = 1.0f / s;
    const float trs = tau * (ROT ? r * 0.0625f : r);
    int8_t* dst = q + (int64_t)row * ldq + (int64_t)blk * 256;
    // F6: the codes of four chunks as floats (exact integers of [-7, 7], +0
    // for zero), converted to E2M3 fields together by the matrix-format
    // conversion; its two 16-value operands interleave (field 2j from the
    // first, 2j + 1 from the second), so code k of the 32 goes to operand k % 2
    f32x16 f6a, f6b;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = i * 4 + ql;
        if (!ROT && blk * 256 + c * E >= K) continue;
        // Fast codes for the chunk; one test of the largest |d| decides
        // whether any element of the chunk needs the exact path.
        uint32_t code[E];
        float fcode[E];   // the same codes as floats (F6 only; n is t - kMagic exactly, +0 for zero)
        float dmax = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float w = v[i * E + e];
            const float t = __builtin_fmaf(w, trs, kMagic);
            const float n = t - kMagic;
            const float d = __builtin_fmaf(w, trs, -n);
            dmax = __builtin_fmaxf(dmax, __builtin_fabsf(d));
            code[e] = f_bits(t);
            fcode[e] = n;
        }
        if (__builtin_expect(mode != 1 || dmax >= kFastMargin, 0)) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float w = v[i * E + e];
                const float t = __builtin_fmaf(w, trs, kMagic);
                const float n = t - kMagic;
                const float d = __builtin_fmaf(w, trs, -n);
                if (mode != 1 || __builtin_fabsf(d) >= kFastMargin) {
                    code[e] = mode == 0 ? 0u : exact_code<ROT, QMAX>(w, tau, s);
                    fcode[e] = (float)(int)(int8_t)(uint8_t)code[e];
                }
            }
        }
        if (F6 && E == 8) {
            static_assert(!F6 || (ROT && QMAX == 7), "FP6 codes are rotated INT4 codes");
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float fc = fcode[e];
                const int k = 8 * (i & 3) + e;
                if (k % 2 == 0) f6a[k / 2] = fc;
                else f6b[k / 2] = fc;
            }
            if ((i & 3) != 3) continue;
            const auto f6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(f6a, f6b, 1.0f);
            const int swp = ((row >> 3) ^ (row >> 4)) & 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // chunk i - 3 + j: 48 bits at bit 48 j of the conversion; piece
                // p = (c % 8) / 4 of K block c / 8, piece bytes 6 (c % 4) .. +5,
                // each 2-byte part at its head (bytes < 16) or tail position
                const int cj = (i - 3 + j) * 4 + ql;
                const int kb = cj >> 3, p = (cj >> 2) & 1, o = 6 * (cj & 3);
#pragma unroll
                for (int h = 0; h < 3; ++h) {
                    const int bit = 48 * j + 16 * h;
                    const uint16_t part = (uint16_t)((uint32_t)f6[bit / 32] >> (bit % 32));
                    const int x = o + 2 * h;
                    const int pos = kb * 48 + (x < 16 ? 16 * p + x : 32 + 8 * (p ^ swp) + (x - 16));
                    *reinterpret_cast<uint16_t*>(img + pos) = part;
                }
            }
            continue;
        }
        uint8_t* out = STAGE ? img + c * E : reinterpret_cast<uint8_t*>(dst) + c * E;
        if (E == 8) {
            u32x2 p;
            p[0] = pack4(code[0], code[1], code[2], code[3]);
            p[1] = pack4(code[4 % E], code[5 % E], code[6 % E], code[7 % E]);
            *reinterpret_cast<u32x2*>(out) = p;
        } else {
            const uint32_t p = pack4(code[0], code[1], code[2], code[3]);
            *reinterpret_cast<uint32_t*>(out) = p;
        }
    }
}

template <class In, bool ROT, int QMAX, bool STAGE, int ACT, bool F6 = false, bool SL = false>
hipError_t launch_staged(const void* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                         float* scale, hipStream_t stream, int R, int threads) {
    constexpr int ESZ = 16 / In::E;
    const int nb = (int)((K + 255) / 256);
    const int64_t grid = (M + R - 1) / R;
    const size_t lds = (F6 ? (size_t)(threads / 64) * kF6Wave : STAGE ? (size_t)(threads / 64) * kStageWave : 0) +
                       (UsesLut<ACT, In16<In>::value>::value ? (size_t)kLutBytes : 0);
    const hipError_t e = build_lut<ACT, In16<In>::value>(stream);
    if (e != hipSuccess) return e;
    rotquant_kernel<In, ROT, QMAX, STAGE, ACT, F6, SL><<<dim3((unsigned)grid), dim3(threads), lds, stream>>>(
        static_cast<const uint8_t*>(x), ldx * ESZ, (int)M, (int)K, nb, R, q, ldq, scale);
    return hipGetLastError();
}

template <class In, bool ROT, int QMAX, int ACT = ACT_NONE, bool F6 = false, bool SL = false>
hipError_t launch_typed(const void* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                        float* scale, hipStream_t stream) {
    const int nb = (int)((K + 255) / 256);
    // Rows per workgroup: one quad per (row, block); pick the row count that
    // leaves the fewest idle lanes in whole waves, preferring ~256 threads.
    int R = 1, best_threads = 0;
    double best_waste = 2.0;
    constexpr int MAXT = kMaxThreads<ACT, In16<In>::value>::value;
    const int r0 = nb >= 64 ? 1 : 64 / nb;
    // K-sliced INT8 codes: an even row count keeps both rows of every 128-byte
    // line of a slice (rows 2i, 2i + 1) in one workgroup
    for (int pass = (SL && !F6) ? 0 : 1; pass < 2 && best_threads == 0; ++pass) {
        for (int r = r0; r <= 2 * r0 + (pass == 0) && 4 * r * nb <= MAXT; ++r) {
            if (pass == 0 && (r & 1)) continue;
            const int th = (4 * r * nb + 63) / 64 * 64;
            const double waste = (double)(th - 4 * r * nb) / th;
            if (waste < best_waste - 1e-9) { best_waste = waste; R = r; best_threads = th; }
        }
    }
    if (best_threads == 0) { R = 1; best_threads = (4 * nb + 63) / 64 * 64; }
    if (R > M) { R = (int)M; best_threads = (4 * R * nb + 63) / 64 * 64; }
    if (best_threads > MAXT) return hipErrorInvalidValue;   // rows longer than the caller's checks allow
    if constexpr (F6)
        return launch_staged<In, ROT, QMAX, true, ACT, true, SL>(x, M, K, ldx, q, ldq, scale, stream, R, best_threads);
    else if constexpr (ROT)
        return launch_staged<In, ROT, QMAX, true, ACT, false, SL>(x, M, K, ldx, q, ldq, scale, stream, R,
                                                                 best_threads);
    else
        return launch_staged<In, ROT, QMAX, false, ACT>(x, M, K, ldx, q, ldq, scale, stream, R, best_threads);
}

}  // namespace

hipError_t launch_rotquant(const void* x, int dtype, bool rotate, int qmax, int64_t M, int64_t K,
                           int64_t ldx, int8_t* q, int64_t ldq, float* scale, hipStream_t stream, int act) {
#define QD_DISPATCH(IN)                                                                       \
    if (rotate) {                                                                             \
        if (qmax == 7) return launch_typed<IN, true, 7>(x, M, K, ldx, q, ldq, scale, stream); \
        return launch_typed<IN, true, 127>(x, M, K, ldx, q, ldq, scale, stream);              \
    }                                                                                         \
    return launch_typed<IN, false, 127>(x, M, K, ldx, q, ldq, scale, stream);
// INT8 codes with an input activation: 16-bit inputs only (checked by the caller).
#define QD_DISPATCH_ACT(IN, A)                                                                \
    if (rotate) return launch_typed<IN, true, 127, A>(x, M, K, ldx, q, ldq, scale, stream);   \
    return launch_typed<IN, false, 127, A>(x, M, K, ldx, q, ldq, scale, stream);
#define QD_DISPATCH_ACTS(IN)                                                                  \
    switch (act) {                                                                            \
        case ACT_GELU_TANH: QD_DISPATCH_ACT(IN, ACT_GELU_TANH)                                \
        case ACT_GELU_ERF: QD_DISPATCH_ACT(IN, ACT_GELU_ERF)                                  \
        case ACT_SILU: QD_DISPATCH_ACT(IN, ACT_SILU)                                          \
        default: QD_DISPATCH_ACT(IN, ACT_RELU)                                                \
    }
    if (act != ACT_NONE) {
        if (dtype == 1) { QD_DISPATCH_ACTS(InBF16) }
        QD_DISPATCH_ACTS(InF16)
    }
    switch (dtype) {
        case 0: QD_DISPATCH(InF32)
        case 1: QD_DISPATCH(InBF16)
        default: QD_DISPATCH(InF16)
    }
#undef QD_DISPATCH
#undef QD_DISPATCH_ACT
#undef QD_DISPATCH_ACTS
}

namespace {

// The activation alone, by the quantizer's code path (table or FP64).
template <int ACT, int IN16>
__global__ __launch_bounds__(256) void act_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                  uint16_t* __restrict__ out) {
    const uint16_t* lut = g_act_lut[(ACT > 0 && ACT < 4) ? ACT - 1 : 0];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t b = x[i];
        if (UsesLut<ACT, IN16>::value) {
            out[i] = (uint16_t)act_bf16_lut(b, lut);
            continue;
        }
        float f;
        if (IN16 == 1) f = bits_f(b << 16);
        else f = (float)__builtin_bit_cast(_Float16, (uint16_t)b);
        const float a = input_act<ACT, IN16>(f);
        // a is exactly representable in the 16-bit type
        out[i] = IN16 == 1 ? (uint16_t)(f_bits(a) >> 16) : __builtin_bit_cast(uint16_t, (_Float16)a);
    }
}

template <int IN16>
hipError_t launch_act16(const void* x, int64_t n, int act, void* out, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    const uint16_t* xi = static_cast<const uint16_t*>(x);
    uint16_t* o = static_cast<uint16_t*>(out);
    hipError_t e = hipSuccess;
    switch (act) {
        case ACT_GELU_TANH: e = build_lut<ACT_GELU_TANH, IN16>(stream); break;
        case ACT_GELU_ERF: e = build_lut<ACT_GELU_ERF, IN16>(stream); break;
        case ACT_SILU: e = build_lut<ACT_SILU, IN16>(stream); break;
        default: break;
    }
    if (e != hipSuccess) return e;
    switch (act) {
        case ACT_GELU_TANH: act_kernel<ACT_GELU_TANH, IN16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(xi, n, o); break;
        case ACT_GELU_ERF: act_kernel<ACT_GELU_ERF, IN16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(xi, n, o); break;
        case ACT_SILU: act_kernel<ACT_SILU, IN16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(xi, n, o); break;
        case ACT_RELU: act_kernel<ACT_RELU, IN16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(xi, n, o); break;
        default: act_kernel<ACT_NONE, IN16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(xi, n, o); break;
    }
    return hipGetLastError();
}

}  // namespace

// Rotated INT8 codes in the K-sliced layout (byte (m, k) at (k / 64) * M * 64 + m * 64 + k % 64).
hipError_t launch_rotquant_sliced(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                  float* scale, hipStream_t stream, int act) {
    const int64_t plane = M * 64;
#define QD_SLICED(IN, A) return launch_typed<IN, true, 127, A, false, true>(x, M, K, ldx, q, plane, scale, stream);
#define QD_SLICED_ACTS(IN)                          \
    switch (act) {                                  \
        case ACT_GELU_TANH: QD_SLICED(IN, ACT_GELU_TANH) \
        case ACT_GELU_ERF: QD_SLICED(IN, ACT_GELU_ERF)   \
        case ACT_SILU: QD_SLICED(IN, ACT_SILU)           \
        case ACT_RELU: QD_SLICED(IN, ACT_RELU)           \
        default: QD_SLICED(IN, ACT_NONE)                 \
    }
    if (dtype == 0) QD_SLICED(InF32, ACT_NONE)
    if (dtype == 1) { QD_SLICED_ACTS(InBF16) }
    QD_SLICED_ACTS(InF16)
#undef QD_SLICED
#undef QD_SLICED_ACTS
}

hipError_t launch_rotquant_fp6(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q6,
                               int64_t ld6, float* scale, hipStream_t stream, bool sliced) {
    int8_t* q = reinterpret_cast<int8_t*>(q6);
    if (sliced) {
        const int64_t plane = M * 96;
        if (dtype == 1) return launch_typed<InBF16, true, 7, ACT_NONE, true, true>(x, M, K, ldx, q, plane, scale, stream);
        return launch_typed<InF16, true, 7, ACT_NONE, true, true>(x, M, K, ldx, q, plane, scale, stream);
    }
    if (dtype == 1) return launch_typed<InBF16, true, 7, ACT_NONE, true>(x, M, K, ldx, q, ld6, scale, stream);
    return launch_typed<InF16, true, 7, ACT_NONE, true>(x, M, K, ldx, q, ld6, scale, stream);
}

hipError_t launch_input_act(const void* x, int dtype, int64_t n, int act, void* out, hipStream_t stream) {
    return dtype == 1 ? launch_act16<1>(x, n, act, out, stream) : launch_act16<2>(x, n, act, out, stream);
}

}  // namespace qd
