// INT8 attention for gfx950 (CDNA4).
//
// int8_attention (comfy-kitchen's INT8-quantized attention behind ComfyUI's
// --use-ck-attention; the ai-jitan-hub article on ComfyUI v0.32.0 says that
// q, k and v are quantized to INT8 and that only the CUDA and HIP backends
// implement it, and gives no formula).  This library's reading: q, k and v
// are quantized per token (one row of D values per head) by the unrotated
// row quantizer of the linear layer; scores are the exact INT32 dot products
// of the codes scaled by sq[i] * sk[j] * scale; softmax over the keys; the
// output row is sum_j p[i][j] * sv[j] * v[j] / sum_j p[i][j], stored as BF16.
//
// attn_i8_kernel: a workgroup of 12 waves (three per SIMD) takes 384 queries of
// one (batch, head), each wave 32 queries, and walks the keys in blocks of 64
// through four LDS stages (flash-attention style: running reference maximum
// and sum, the output accumulators rescaled only when some query's maximum
// outgrew its reference by more than 2^8).  Block kb + 2 is staged during
// block kb, so one workgroup barrier per two blocks keeps every stage
// written before it is read and read before it is rewritten; between
// barriers the waves of a SIMD drift apart and overlap their phases.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_i32_32x32x32_i8 (K from LDS as the "A" operand, the wave's Q
//    codes in registers as "B"), so a lane holds 16 keys of ONE query: the
//    row maximum and sum need one exchange between the two half-waves.  The
//    key scale is applied to the scores, the query scale (>= 0, with the
//    softmax scale and log2(e)) inside the base-2 exponent's FMA.
//  * The probabilities are rounded to BF16 in registers and are directly the
//    "B" operand of v_mfma_f32_32x32x16_bf16 computing O^T = V^T P^T: the
//    key order inside each 16-key step is the one the score layout leaves in
//    the lanes, and the V^T operand is read in the same order from a
//    transposed tile of dequantized values sv[key] * vc[key][d] rounded to
//    BF16, written into LDS 4 keys x 4 dims per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qd_device.h"
#include "qd_launch.h"

namespace qd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// max(x, x of lane ^ 32): the two half-waves exchange through
// v_permlane32_swap (a VALU lane swap, no LDS round trip); the s_nop pads
// cover the VALU write -> swap -> VALU read hazards
__device__ __forceinline__ float max_xor32(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1" : "+v"(a), "+v"(b));
    return a;
}

constexpr int AW = 12;               // waves per workgroup, 32 queries each
constexpr int AQ = 32 * AW;          // queries per workgroup
constexpr int AK = 64;               // keys per block
constexpr int VT_STRIDE = AK + 4;    // BF16 per row of the transposed value tile (136 bytes)
constexpr int ATT_THREADS = 64 * AW;

template <int D>
struct AttnStage {
    int8_t k[AK * D];                // key codes, 16-byte chunks of row r XOR-swizzled by (r / (256 / D)) % (D / 16)
    uint16_t vt[D * VT_STRIDE];      // dequantized values sv[key] * vc[key][d] as BF16, transposed: vt[d][key]
    float sk[AK];
};

template <int D>
__global__ __launch_bounds__(ATT_THREADS, 3) void attn_i8_kernel(const int8_t* __restrict__ qc,
                                                              const float* __restrict__ sq,
                                                              const int8_t* __restrict__ kc,
                                                              const float* __restrict__ sk,
                                                              const int8_t* __restrict__ vc,
                                                              const float* __restrict__ sv,
                                                              uint16_t* __restrict__ out, int Lq, int Lk,
                                                              float c) {
    constexpr int NS = D / 32;                   // 32-element steps along D (score MFMA K, output tiles)
    constexpr int CPR = D / 16;                  // 16-byte chunks per key row
    constexpr int KCH = (AK * CPR + ATT_THREADS - 1) / ATT_THREADS;   // key chunks staged per thread
    constexpr int VG = AK / 4 * D / 4;           // value groups of 4 keys x 4 dims
    // chunk swizzle of a key row: 256 bytes of LDS banks hold 256 / D rows, so
    // rows r and r + 256 / D share banks; XOR the chunk with the row's next bits
    // to put the 16 rows read by 16 lanes on 16 distinct 16-byte bank groups
    auto kswz = [](int row) { return (row / (256 / D)) & (CPR - 1); };
    constexpr int NST = 4, PB = 2;   // LDS stages; blocks per barrier (= staging distance in blocks)
    __shared__ AttnStage<D> st[NST];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int fr = lane & 31;
    const int h = lane >> 5;
    // Workgroups are dispatched to the 8 XCDs round-robin in launch order;
    // renumber them so that each XCD takes a contiguous range of (head, query
    // block) pairs, i.e. whole heads, whose keys and values its L2 then serves
    // to all of that head's query blocks.
    const int nqb = (int)gridDim.x;
    const int Gt = nqb * (int)gridDim.y;
    const int gl = (int)blockIdx.x + nqb * (int)blockIdx.y;
    const int xc = gl % 8;
    const int tl = xc * (Gt / 8) + min(xc, Gt % 8) + gl / 8;
    const int qb = tl % nqb, hd = tl / nqb;
    const int64_t qbase = (int64_t)hd * Lq;
    const int64_t kbase = (int64_t)hd * Lk;
    const int q_row = qb * AQ + wave * 32 + fr;   // this lane's query
    const int qr = min(q_row, Lq - 1);

    i32x4 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = *reinterpret_cast<const i32x4*>(qc + (qbase + qr) * D + 32 * s + 16 * h);
    const float sqc = sq[qbase + qr] * c;   // >= 0: applied inside the exponent

    // staging of key block kb: registers first (loads in flight during the
    // math of block kb - PB), then LDS.  Value group vg: keys 4 (vg % 16) + 0..3,
    // dims 4 (vg / 16) + 0..3.
    constexpr int VGI = (VG + ATT_THREADS - 1) / ATT_THREADS;   // value groups staged per thread
    u32x4 kreg[KCH];
    uint32_t vreg[VGI][4];
    float vscale[VGI][4];
    float skr = 0.0f;
    auto gload = [&](int kb) {
        const int k0 = kb * AK;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tid + ATT_THREADS * i;
            if (ch < AK * CPR) {
                const int key = min(k0 + ch / CPR, Lk - 1);
                kreg[i] = *reinterpret_cast<const u32x4*>(kc + (kbase + key) * D + (ch % CPR) * 16);
            }
        }
#pragma unroll
        for (int i = 0; i < VGI; ++i) {
            const int vg = tid + ATT_THREADS * i;
            if (vg < VG) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = min(k0 + 4 * (vg & 15) + j, Lk - 1);
                    vreg[i][j] = *reinterpret_cast<const uint32_t*>(vc + (kbase + key) * D + 4 * (vg >> 4));
                    vscale[i][j] = sv[kbase + key];
                }
            }
        }
        if (tid < AK) skr = sk[kbase + min(k0 + tid, Lk - 1)];
    };
    auto sstore = [&](AttnStage<D>& S) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tid + ATT_THREADS * i;
            if (ch < AK * CPR) {
                const int row = ch / CPR;
                *reinterpret_cast<u32x4*>(S.k + row * D + (((ch % CPR) ^ kswz(row)) << 4)) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < VGI; ++i) {
            const int vg = tid + ATT_THREADS * i;
            if (vg < VG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {      // dim 4 (vg / 16) + e: keys 4 (vg % 16) .. +3
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        f[j] = (float)(int8_t)((vreg[i][j] >> (8 * e)) & 0xFFu) * vscale[i][j];
                    const u32x2 pk = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
                    *reinterpret_cast<u32x2*>(S.vt + (4 * (vg >> 4) + e) * VT_STRIDE + 4 * (vg & 15)) = pk;
                }
            }
        }
        if (tid < AK) S.sk[tid] = skr;
    };

    f32x16 o[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.0f;
    float m_run = -__builtin_inff();   // running maximum of acc * sk (the query's scale applied later)
    float l_run = 0.0f;

    const int nkb = (Lk + AK - 1) / AK;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        gload(j);
        sstore(st[j]);
    }
    __syncthreads();
    // key blocks: the full ones, then the partial last one (keys past Lk
    // masked) as a separate instance so that the full blocks carry no masking
    auto block = [&](int kb, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const AttnStage<D>& S = st[kb % NST];
        gload(kb + PB);   // rows clamped to Lk - 1 past the last block

        // S^T tiles: keys kt*32 + 8g + 4h + e (element 4g + e), query fr; the
        // two tiles' MFMAs alternate (independent accumulators).  The wave
        // issues them at raised priority: the block's softmax waits on them.
        __builtin_amdgcn_s_setprio(1);
        i32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int row = kt * 32 + fr;
                const i32x4 kf =
                    *reinterpret_cast<const i32x4*>(S.k + row * D + (((2 * s + h) ^ kswz(row)) << 4));
                sacc[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], sacc[kt], 0, 0, 0);
            }
        }

        __builtin_amdgcn_s_setprio(0);
        float t[2][16];
        float bm = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 skv = *reinterpret_cast<const f32x4*>(S.sk + kt * 32 + 8 * g + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = (float)sacc[kt][4 * g + e] * skv[e];
                    if (TAIL) x = kb * AK + kt * 32 + 8 * g + 4 * h + e < Lk ? x : -__builtin_inff();
                    t[kt][4 * g + e] = x;
                    bm = __builtin_fmaxf(bm, x);
                }
            }
        }
        bm = max_xor32(bm);
        // The reference maximum only moves when the block's maximum exceeds it
        // by more than 2^8 in the exponent (the probabilities stay <= 256, far
        // inside FP32 and BF16 range, and out = sum p v / sum p does not depend
        // on the reference), so the rescale below is rare after the first blocks.
        const bool grow = m_run == -__builtin_inff() || (bm - m_run) * sqc > 8.0f;
        if (__any(grow)) {
            // the first block: nothing accumulated yet (also avoids -inf * 0 for a zero query)
            const float alpha = !grow ? 1.0f
                                : m_run == -__builtin_inff() ? 0.0f
                                : __builtin_amdgcn_exp2f((m_run - bm) * sqc);
            m_run = grow ? bm : m_run;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NS; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        const float nm = -m_run * sqc;

        // p as BF16: 16-key step s16 = 2 kt + g / 2 holds keys 16 s16 + 8 (g % 2) + 4h + e
        // at element 4 (g % 2) + e.  O^T tiles: dims dt*32 + 8g + 4h + e (element
        // 4g + e), query fr.  The first tile's probabilities go to the matrix
        // cores before the second tile's are computed, so that this VALU work
        // (and the next block's staging) issues while those MFMAs run.
        float ls = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            u32x4 pb[2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kt][4 * g + e], sqc, nm));
                    // keys past Lk (tail block only): p = 0, also for a zero query (-inf * 0)
                    if (TAIL) pv[e] = kb * AK + kt * 32 + 8 * g + 4 * h + e < Lk ? pv[e] : 0.0f;
                    ls += pv[e];
                }
                pb[g / 2][2 * (g % 2)] = pack_bf16x2(pv[0], pv[1]);
                pb[g / 2][2 * (g % 2) + 1] = pack_bf16x2(pv[2], pv[3]);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int s16 = 2 * kt + s2;
                const bf16x8 bop = __builtin_bit_cast(bf16x8, pb[s2]);
#pragma unroll
                for (int dt = 0; dt < NS; ++dt) {
                    const uint16_t* vrow = S.vt + (dt * 32 + fr) * VT_STRIDE + 16 * s16 + 4 * h;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
                    const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bop, o[dt], 0,
                                                                    0, 0);
                }
            }
        }
        l_run += ls;
        // staging of block kb + PB (past the last block it reloads clamped rows
        // into stages nobody reads any more: no branch, one scheduling region)
        sstore(st[(kb + PB) % NST]);
        // schedule: value-tile reads first, the first tile's probabilities, then
        // each of its MFMAs followed by a share of the remaining VALU work
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * 4 * NS, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
#pragma unroll
        for (int i = 0; i < 2 * NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NS, 0);


        if (kb % PB == PB - 1) __syncthreads();
    };
    const int nfull = Lk / AK;
    for (int kb = 0; kb < nfull; ++kb) block(kb, std::false_type{});
    if (nfull < nkb) block(nfull, std::true_type{});

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (q_row < Lq) {
        uint16_t* orow = out + (qbase + q_row) * D;
#pragma unroll
        for (int dt = 0; dt < NS; ++dt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 pk = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                  pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * g + 4 * h) = pk;
            }
        }
    }
}

template <int D>
hipError_t launch_attn(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk, const int8_t* vc,
                       const float* sv, uint16_t* out, int64_t BH, int64_t Lq, int64_t Lk, float c,
                       hipStream_t stream) {
    const dim3 grid((unsigned)((Lq + AQ - 1) / AQ), (unsigned)BH);
    attn_i8_kernel<D><<<grid, dim3(ATT_THREADS), 0, stream>>>(qc, sq, kc, sk, vc, sv, out, (int)Lq, (int)Lk, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_i8(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                               const int8_t* vc, const float* sv, void* out, int64_t BH, int64_t Lq, int64_t Lk,
                               int64_t D, float scale, hipStream_t stream) {
    const float c = scale * 1.4426950408889634f;   // log2(e): the kernel exponentiates in base 2
    uint16_t* o = static_cast<uint16_t*>(out);
    if (D == 64) return launch_attn<64>(qc, sq, kc, sk, vc, sv, o, BH, Lq, Lk, c, stream);
    return launch_attn<128>(qc, sq, kc, sk, vc, sv, o, BH, Lq, Lk, c, stream);
}

}  // namespace qd
