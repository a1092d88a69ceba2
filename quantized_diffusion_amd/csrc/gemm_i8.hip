// INT8 x INT8 -> INT32 GEMM on the gfx950 matrix cores with a fused
// dequantizing epilogue.
//
// Computes acc[m, n] = sum_k aq[m, k] * wq[n, k] (both operands K-contiguous,
// "TN") exactly in INT32 and, in the BF16 mode, writes
// y[m, n] = bf16_rne(((float)acc * a_scale[m]) * w_scale[n] + bias[n])
// straight from the accumulators, so the INT32 product never reaches memory
// (the fused rescale-and-bias store of the ComfyUI-AppleSilicon-FP8 README,
// "What it fixes" row 17; dtypes per the SGLang PR "Tune Kitchen INT8 row
// splitting for SM120", "Accuracy Test").  The INT32 mode stores the raw
// accumulators instead and exists to verify the contraction bit for bit.
//
// Main kernel (K % 64 == 0): a workgroup of 8 waves owns a 256 x 256 output
// tile; each wave owns 64 output columns x 128 rows in eight
// v_mfma_i32_32x32x32_i8 accumulators, two waves per SIMD so that one keeps
// the matrix pipe fed while the other waits.  Operands move global -> LDS
// with global_load_lds_dwordx4 (no staging registers) through a ring of
// four 64-byte K slices; copies run three slices ahead and are spread over
// the slice so that the copy queue never stalls a wave for long.  The output
// tile is staged through the ring so that every store writes whole rows; a
// whole tile stores through a wave-uniform row base plus fixed 32-bit lane
// offsets (no per-store bounds checks or 64-bit address arithmetic), and
// without bias the epilogue adds -0, which changes no value, instead of
// selecting per output.
// A wide variant owns 256 x 384 output tiles (twelve accumulators per wave,
// four 40 KB stages), moving 17 % fewer bytes from L2 into LDS per MAC; the
// launcher picks the tile by shape (rounds of one workgroup per CU).
// A general kernel (any K % 16 == 0) stages operands through registers.
// The K loops of the eight-wave kernels run in two phases: a steady phase
// for every slice that has the whole ring after it (all copies issued, a
// fixed number of slices left in flight, no run-time conditions in the loop
// body), then the last slices with the conditions; the fewer scalar
// instructions per slice raised the INT8 kernel's MFMA issue rate per clock
// by about a tenth and the FP6 kernel's by almost half.
// The eight-wave kernels take a row stride and a K-slice stride per operand,
// so they read row-major operands or the K-sliced layout (each 64-byte K
// slice of all rows stored contiguously: a copy instruction then reads 1 KB
// of consecutive bytes, whole 128-byte lines, at lower power per byte).
// Copy sources are a wave-uniform base in SGPRs (advanced by a scalar add
// per slice) plus a fixed 32-bit offset per lane, so the loops spend no
// vector instructions on addresses; the boundary keeps operand row strides
// at most QD_MAX_LD_GEMM so that a tile's offsets fit 32 bits.
// The FP6 kernel (W4A4 codes as FP6 E2M3) is described before its code.
//
// MFMA roles.  The weight tile is the MFMA "A" operand (its rows index n)
// and the activation tile is "B" (its columns index m), so each lane ends up
// holding four consecutive n of one m per 4-register group.  A lane feeds
// row (lane % 32) of either operand with the 16 bytes of K-group (lane / 32);
// both operands use the same byte order, so the dot product is exact
// whatever order the hardware assigns within a K-group.
//
// LDS layout.  Each operand stage is [256 rows][64 bytes]; the four 16-byte
// chunks of row r are stored XOR-swizzled by ((r >> 1) ^ (r >> 2)) & 3 so
// that the 16-byte reads of 32 consecutive rows hit distinct banks.
//
// Tile order.  Workgroup g runs on XCD g % 8; tiles are renumbered so that
// each XCD gets a contiguous range, and inside a range tiles go down groups
// of GROUP_M tile rows first, so the ~32 tiles an XCD runs at once share
// A and B panels in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qd_device.h"
#include "qd_launch.h"

namespace qd {
namespace {

constexpr int BM = 256;      // activation rows per tile
constexpr int BN = 256;      // weight rows (output columns) per tile
constexpr int BK = 64;       // K bytes per slice
constexpr int NT = 256;      // threads per workgroup
constexpr int GROUP_M = 8;   // tile rows per L2 group
constexpr int NXCD = 8;

enum { MODE_BF16 = 0, MODE_I32 = 1 };

struct EpiArgs {
    const float* a_scale;
    const float* w_scale;
    const uint16_t* bias;   // may be null
    void* out;              // uint16_t (BF16) or int32_t
    int64_t ldo;            // elements
    int a_step;             // 1: a_scale[m]; 0: a_scale[0] for every row
    int w_step;             // 1: w_scale[n]; 0: w_scale[0] for every column
};

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_f((uint32_t)b << 16); }

// Four outputs y[m, n + e] = bf16_rne(((float)acc_e * sx) * sw_e + b_e), FP32, no contraction.
__device__ __forceinline__ void store_bf16x4(const int32_t* a4, float sx, int n, int N, int64_t m,
                                             const EpiArgs& ep) {
#pragma clang fp contract(off)
    uint16_t* dst = static_cast<uint16_t*>(ep.out) + m * ep.ldo + n;
    if (n + 3 < N) {
        const f32x4 sw = ep.w_step ? *reinterpret_cast<const f32x4*>(ep.w_scale + n)
                                   : f32x4{ep.w_scale[0], ep.w_scale[0], ep.w_scale[0], ep.w_scale[0]};
        float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ep.bias) {
            const u32x2 bb = *reinterpret_cast<const u32x2*>(ep.bias + n);
            b4[0] = bits_f(bb[0] << 16);
            b4[1] = bits_f(bb[0] & 0xFFFF0000u);
            b4[2] = bits_f(bb[1] << 16);
            b4[3] = bits_f(bb[1] & 0xFFFF0000u);
        }
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float tt = (float)a4[e];
            tt = tt * sx;
            tt = tt * sw[e];
            if (ep.bias) tt = tt + b4[e];
            o[e] = tt;
        }
        u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
        for (int e = 0; e < 4 && n + e < N; ++e) {
            float tt = (float)a4[e];
            tt = tt * sx;
            tt = tt * ep.w_scale[(n + e) * ep.w_step];
            if (ep.bias) tt = tt + bf16_to_f32(ep.bias[n + e]);
            dst[e] = (uint16_t)(pack_bf16x2(tt, 0.0f) & 0xFFFFu);
        }
    }
}

// Four outputs bf16_rne(((float)acc_e * sx) * sw_e + b_e) packed as BF16 pairs; the
// bias arrives widened to FP32 (exact), once per tile column in LDS.
__device__ __forceinline__ u32x2 epi_bf16x4(const int32_t* a4, float sx, const f32x4& sw, const f32x4& b,
                                            bool has_bias) {
#pragma clang fp contract(off)
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float tt = (float)a4[e];
        tt = tt * sx;
        tt = tt * sw[e];
        if (has_bias) tt = tt + b[e];
        o[e] = tt;
    }
    u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    return pk;
}

__device__ __forceinline__ void store_i32x4(const int32_t* a4, int n, int N, int64_t m,
                                            const EpiArgs& ep) {
    int32_t* dst = static_cast<int32_t*>(ep.out) + m * ep.ldo + n;
    if (n + 3 < N) {
        i32x4 v = {a4[0], a4[1], a4[2], a4[3]};
        *reinterpret_cast<i32x4*>(dst) = v;
    } else {
        for (int e = 0; e < 4 && n + e < N; ++e) dst[e] = a4[e];
    }
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void gemm_i8_kernel(const int8_t* __restrict__ A, int64_t lda,
                                                        const int8_t* __restrict__ W, int64_t ldw,
                                                        int M, int N, int K, EpiArgs ep) {
    __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t sW[2][BN * BK];

    // ---- tile coordinates (XCD-contiguous, grouped) ----
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int T = tiles_m * tiles_n;
    const int g = blockIdx.x;
    const int xcd = g % NXCD;
    const int q8 = T / NXCD, rem = T % NXCD;
    const int t = xcd * q8 + min(xcd, rem) + g / NXCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = t / per_group;
    const int first_m = group * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tg = t - group * per_group;
    const int tm = first_m + tg % gsz;
    const int tn = tg / gsz;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // 128-row half of the activation tile
    const int wn = wave >> 1;  // 128-row half of the weight tile

    // ---- global -> register staging: 4 chunks per operand per thread ----
    // chunk id q = i*256 + tid -> row q/4, 16-byte column q%4
    const int ld_c = tid & 3;
    const int ld_r = tid >> 2;     // + 64*i
    const int8_t* a_src[4];
    const int8_t* w_src[4];
    bool a_ok[4], w_ok[4];
    int st_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ld_r + 64 * i;
        a_ok[i] = (m0 + r) < M;
        w_ok[i] = (n0 + r) < N;
        a_src[i] = A + (int64_t)(a_ok[i] ? m0 + r : 0) * lda + ld_c * 16;
        w_src[i] = W + (int64_t)(w_ok[i] ? n0 + r : 0) * ldw + ld_c * 16;
        st_off[i] = r * BK + ((ld_c ^ swz(r)) << 4);
    }
    u32x4 ra[4], rw[4];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
        const bool kin = (k0 + ld_c * 16) < K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = (a_ok[i] && kin) ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : zero4;
            rw[i] = (w_ok[i] && kin) ? *reinterpret_cast<const u32x4*>(w_src[i] + k0) : zero4;
        }
    };
    auto sstore = [&](int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4*>(&sA[s][st_off[i]]) = ra[i];
            *reinterpret_cast<u32x4*>(&sW[s][st_off[i]]) = rw[i];
        }
    };

    // ---- LDS -> MFMA operand offsets ----
    // wave reads rows base + 32*blk + lane%32, chunk 2*kk + lane/32
    const int fr = lane & 31;
    const int fk = lane >> 5;
    int a_off[4][2], w_off[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int ra_row = wm * 128 + b * 32 + fr;
        const int rw_row = wn * 128 + b * 32 + fr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = 2 * kk + fk;
            a_off[b][kk] = ra_row * BK + ((c ^ swz(ra_row)) << 4);
            w_off[b][kk] = rw_row * BK + ((c ^ swz(rw_row)) << 4);
        }
    }

    i32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            i32x4 fa[4], fw[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                fw[b] = *reinterpret_cast<const i32x4*>(&sW[s][w_off[b][kk]]);
                fa[b] = *reinterpret_cast<const i32x4*>(&sA[s][a_off[b][kk]]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i], fa[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(s ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    // acc[i][j][4*g4 + e] holds (n, m) = (n0 + wn*128 + 32*i + 8*g4 + 4*fk + e,
    //                                     m0 + wm*128 + 32*j + fr)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 128 + 32 * j + fr;
        if (m >= M) continue;
        const float sx = (MODE == MODE_BF16) ? ep.a_scale[m * ep.a_step] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + wn * 128 + 32 * i + 8 * g4 + 4 * fk;
                if (n >= N) continue;
                const int32_t a4[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                       acc[i][j][4 * g4 + 3]};
                if (MODE == MODE_I32) store_i32x4(a4, n, N, m, ep);
                else store_bf16x4(a4, sx, n, N, m, ep);
            }
        }
    }
}

typedef __attribute__((address_space(3))) int8_t lds_i8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_i8*)p;
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// wait until at most `groups` slices' copies (PER per thread each) are in flight
template <int PER>
__device__ __forceinline__ void wait_groups(int groups) {
    switch (groups) {
        case 0:
        case -1: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<PER>(); break;
        case 2: wait_vmcnt<2 * PER>(); break;
        default: wait_vmcnt<3 * PER>(); break;
    }
}

// the same with EXTRA further loads issued after the last copy (still in flight)
template <int PER, int EXTRA>
__device__ __forceinline__ void wait_groups_x(int groups) {
    switch (groups) {
        case 0:
        case -1: wait_vmcnt<EXTRA>(); break;
        case 1: wait_vmcnt<PER + EXTRA>(); break;
        case 2: wait_vmcnt<2 * PER + EXTRA>(); break;
        default: wait_vmcnt<3 * PER + EXTRA>(); break;
    }
}

// 16 signed INT4 codes packed two per byte (code 2i in the low nibble of
// byte i) -> 16 INT8 bytes in code order.  Byte-wise sign extension of a
// nibble v: ((v ^ 8) + 0x78) ^ 0x80, which never carries across bytes.
__device__ __forceinline__ i32x4 unpack_int4x16(const u32x2& p) {
    i32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t lo = p[h] & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 of this word
        uint32_t hi = (p[h] >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
        lo = ((lo ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
        hi = ((hi ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
        r[2 * h] = (int32_t)__builtin_amdgcn_perm(hi, lo, 0x05010400u);
        r[2 * h + 1] = (int32_t)__builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
    return r;
}

// 16-byte global -> LDS copy per lane.  The source is split into a wave-uniform
// base in SGPRs (the tile's first row plus the slice offset: one scalar add per
// slice) and a fixed per-lane 32-bit offset (row within the tile x row pitch +
// chunk; below 2^32 because tiles have at most 384 rows and K <= QD_MAX_K_GEMM),
// so the K loop spends no vector instructions on copy addresses.
__device__ __forceinline__ void dma16s(uint32_t lds, uint32_t voff, const int8_t* sbase) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// ---------------------------------------------------------------------------
// Main kernel (K % 64 == 0).  Per K slice t a wave
//   1. issues the LDS reads of slice t's second K half and the MFMAs of the
//      first half (operands already in registers), plus its two weight-row
//      copies of slice t+NS-1, one per four MFMAs;
//   2. drains its LDS reads, waits until its own copies of slice t+1 have
//      landed, and meets the other waves at one barrier: after it slice t+1
//      is visible to all and nobody reads stage t any more;
//   3. issues the LDS reads of slice t+1's first half and the MFMAs of slice
//      t's second half, plus its two activation-row copies of slice t+NS
//      into stage t.
// The copies are issued from inline assembly so that the compiler does not
// drain them at every barrier; their completion is awaited explicitly with
// s_waitcnt vmcnt.  Each copy instruction moves 1 KB (64 lanes x 16 B) into
// consecutive LDS bytes: 16 rows of 64 bytes, a lane fetching the chunk that
// belongs at its swizzled slot.  Rows past M or N re-read the last valid row
// (their outputs are never stored).  The tile's row scales, column scales
// and bias are copied into LDS above the ring during the prologue.
constexpr int NT8 = 512;
constexpr int EPI_LDS = 4 * 1024;   // sx[256] f32, sw[256] f32, bias[256] widened to f32 (+pad)

enum { WF_I8 = 0, WF_I4 = 1 };   // weight operand: INT8, or INT4 packed two per byte

// packed-INT4 weight stage: [256 rows][32 bytes], 16-byte chunk c of row r at c ^ ((r >> 3) & 1)
__device__ __forceinline__ int swz4(int row) { return (row >> 3) & 1; }

template <int MODE, int NS, int WF>
__global__ __launch_bounds__(NT8, 1) void gemm_i8_w8_kernel(const int8_t* __restrict__ A, int64_t lda, int64_t a_ss,
                                                           const int8_t* __restrict__ W, int64_t ldw, int64_t w_ss,
                                                           int M, int N, int K, EpiArgs ep) {
    constexpr int WROW = WF == WF_I4 ? BK / 2 : BK;          // weight bytes per row per slice
    constexpr int STG = BM * BK + BN * WROW;                 // bytes per stage
    constexpr int PER = WF == WF_I4 ? 3 : 4;                 // copies per slice per thread
    constexpr int RING = NS * STG > 256 * 512 ? NS * STG : 256 * 512;   // the output tile is staged here too
    __shared__ __attribute__((aligned(1024))) int8_t smem[RING + EPI_LDS];
    float* l_sx = reinterpret_cast<float*>(smem + RING);
    float* l_sw = l_sx + 256;
    float* l_b = l_sw + 256;

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int T = tiles_m * tiles_n;
    const int g = blockIdx.x;
    const int xcd = g % NXCD;
    const int q8 = T / NXCD, rem = T % NXCD;
    const int t_lin = xcd * q8 + min(xcd, rem) + g / NXCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = t_lin / per_group;
    const int first_m = group * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tg = t_lin - group * per_group;
    const int m0 = (first_m + tg % gsz) * BM;
    const int n0 = (tg / gsz) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;    // 128-row half of the activation tile
    const int wn = wave >> 1;   // 64-row quarter of the weight tile

    // epilogue operands of the tile -> LDS (plain loads, consumed after the K loop)
    if (MODE == MODE_BF16) {
        if (tid < 256) {
            const int m = min(m0 + tid, M - 1);
            l_sx[tid] = ep.a_scale[m * ep.a_step];
        } else {
            const int c = tid - 256;
            const int n = min(n0 + c, N - 1);
            l_sw[c] = ep.w_scale[n * ep.w_step];
            // without bias, -0: adding it changes no value (unlike +0, which turns -0 into +0)
            l_b[c] = ep.bias ? bf16_to_f32(ep.bias[n]) : -0.0f;
        }
    }

    // copies: activation instruction i (0, 1) of this wave covers rows
    // 16 * (wave + 8 i) + lane / 4; INT8 weights likewise; packed INT4 weights
    // take one instruction per wave for rows 32 * wave + lane / 2
    // (sources: a uniform tile base advanced per slice plus a fixed per-lane offset)
    uint32_t va[2], vw[2];
    uint32_t lrow[2], lwrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int rt = 16 * (wave + 8 * i) + (lane >> 2);
        const int c = (lane & 3) ^ swz(rt);
        va[i] = (uint32_t)((int64_t)(min(m0 + rt, M - 1) - m0) * lda + c * 16);
        lrow[i] = (uint32_t)(16 * (wave + 8 * i) * BK);
        if (WF == WF_I8) {
            vw[i] = (uint32_t)((int64_t)(min(n0 + rt, N - 1) - n0) * ldw + c * 16);
            lwrow[i] = lrow[i];
        } else {
            const int rw = 32 * wave + (lane >> 1);
            const int cw = (lane & 1) ^ swz4(rw);
            vw[i] = (uint32_t)((int64_t)(min(n0 + rw, N - 1) - n0) * ldw + cw * 16);
            lwrow[i] = (uint32_t)(32 * wave * WROW);
        }
    }
    const int8_t* a_base = A + (int64_t)m0 * lda;
    const int8_t* w_base = W + (int64_t)n0 * ldw;
    const uint32_t lds0 = lds_addr(smem);
    // slice u into LDS stage sg (= u % NS; a constant in the unrolled steady loop)
    auto copy_part = [&](int u, int sg, int part, int i) {
        const uint32_t sb = lds0 + (uint32_t)(sg * STG);
        if (part == 0) dma16s(sb + lrow[i], va[i], a_base + (int64_t)u * a_ss);
        else if (WF == WF_I8 || i == 0) dma16s(sb + BM * BK + lwrow[i], vw[i], w_base + (int64_t)u * w_ss);
    };
    auto issue = [&](int u) {
        copy_part(u, u, 0, 0);
        copy_part(u, u, 0, 1);
        copy_part(u, u, 1, 0);
        copy_part(u, u, 1, 1);
    };

    const int fr = lane & 31;
    const int fk = lane >> 5;
    int a_off[4][2], w_off[2][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int ra_row = wm * 128 + b * 32 + fr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) a_off[b][kk] = ra_row * BK + (((2 * kk + fk) ^ swz(ra_row)) << 4);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int rw_row = wn * 64 + b * 32 + fr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (WF == WF_I8)
                w_off[b][kk] = BM * BK + rw_row * BK + (((2 * kk + fk) ^ swz(rw_row)) << 4);
            else   // 16 codes = 8 packed bytes: chunk kk, half fk
                w_off[b][kk] = BM * BK + rw_row * WROW + ((kk ^ swz4(rw_row)) << 4) + (fk << 3);
        }
    }
    auto rd_a = [&](int sg, int kk, int b, i32x4* fa) {
        fa[b] = *reinterpret_cast<const i32x4*>(smem + sg * STG + a_off[b][kk]);
    };
    auto rd_w = [&](int sg, int kk, int b, i32x4* fw) {
        if (WF == WF_I8) fw[b] = *reinterpret_cast<const i32x4*>(smem + sg * STG + w_off[b][kk]);
        else fw[b] = unpack_int4x16(*reinterpret_cast<const u32x2*>(smem + sg * STG + w_off[b][kk]));
    };

    i32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = K / BK;
    // slices 0 .. NS-2 in flight (4 copies per slice per thread), wait for slice 0
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (u < nk) issue(u);
    wait_groups<PER>(min(nk, NS - 1) - 1);
    __syncthreads();   // slice 0 and the epilogue operands are visible
    if (NS - 1 < nk) {
        copy_part(NS - 1, NS - 1, 0, 0);
        copy_part(NS - 1, NS - 1, 0, 1);
    }

    // The loop runs from barrier to barrier (second half of slice t, then
    // first half of slice t + 1), so that no LDS read is pending at its back edge.
    i32x4 a0[4], w0[2], a1[4], w1[2];
    // STEADY: a slice with NS more after it, where every copy is issued and
    // NS - 2 slices stay in flight (no run-time conditions in the loop body)
    // stage_tag: t % NS when the caller knows it at compile time, else -1
    auto first_half = [&](int t, auto steady_tag, auto stage_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int ST = decltype(stage_tag)::value;
        const int sc = ST >= 0 ? ST : t % NS;                          // slice t
        const int sp = ST >= 0 ? (ST + NS - 1) % NS : (t + NS - 1) % NS;   // slice t + NS - 1
        // first half of slice t; reads of its second half; weight-row copies of slice t+NS-1
        const bool late = STEADY || t + NS - 1 < nk;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            rd_w(sc, 1, q, w1);
            rd_a(sc, 1, 2 * q, a1);
            rd_a(sc, 1, 2 * q + 1, a1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[q][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0[q], a0[j], acc[q][j], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (late) copy_part(t + NS - 1, sp, 1, q);
        }
        acc[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[0], a1[0], acc[0][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (STEADY) wait_vmcnt<(NS - 2) * PER>();
        else wait_groups<PER>(min(nk - 1, t + NS - 1) - (t + 1));
        __builtin_amdgcn_s_barrier();
    };
    auto second_half = [&](int t, bool next, auto steady_tag, auto stage_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int ST = decltype(stage_tag)::value;
        const int sc = ST >= 0 ? ST : t % NS;                   // slice t (and t + NS)
        const int sn = ST >= 0 ? (ST + 1) % NS : (t + 1) % NS;  // slice t + 1
        // second half of slice t; reads of slice t+1's first half; activation-row copies of slice t+NS
        const bool early = STEADY || t + NS < nk;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (next) {
                rd_w(sn, 0, q, w0);
                rd_a(sn, 0, 2 * q, a0);
                rd_a(sn, 0, 2 * q + 1, a0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (q != 0 || j > 0)
                    acc[q][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[q], a1[j], acc[q][j], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (early) copy_part(t + NS, sc, 0, q);
        }
    };
#pragma unroll
    for (int b = 0; b < 4; ++b) rd_a(0, 0, b, a0);
#pragma unroll
    for (int b = 0; b < 2; ++b) rd_w(0, 0, b, w0);
    using rt = std::integral_constant<int, -1>;
    first_half(0, std::false_type{}, std::integral_constant<int, 0>{});
    // steady slices NS at a time, so that each one's LDS stages are constants
    // (no per-slice stage arithmetic or address adds), then the rest
    static_assert(NS == 4 || NS == 5, "the unrolled steady loop covers four or five stages");
    auto steady = [&](int t0, auto jt) {
        constexpr int J = decltype(jt)::value;
        second_half(t0 + J, true, std::true_type{}, std::integral_constant<int, J>{});
        first_half(t0 + J + 1, std::true_type{}, std::integral_constant<int, (J + 1) % NS>{});
    };
    int t = 0;
    for (; t + 2 * NS - 1 < nk; t += NS) {
        steady(t, std::integral_constant<int, 0>{});
        steady(t, std::integral_constant<int, 1>{});
        steady(t, std::integral_constant<int, 2>{});
        steady(t, std::integral_constant<int, 3>{});
        if constexpr (NS == 5) steady(t, std::integral_constant<int, 4 % NS>{});
    }
    for (; t + NS < nk; ++t) {
        second_half(t, true, std::true_type{}, rt{});
        first_half(t + 1, std::true_type{}, rt{});
    }
    for (; t + 1 < nk; ++t) {
        second_half(t, true, std::false_type{}, rt{});
        first_half(t + 1, std::false_type{}, rt{});
    }
    second_half(nk - 1, false, std::false_type{}, rt{});

    if (MODE == MODE_BF16) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        // acc[i][j][4 g4 + e]: (n, m) = (wn*64 + 32 i + 8 g4 + 4 fk + e, wm*128 + 32 j + fr) in the tile
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wm * 128 + 32 * j + fr;
            const float sx = l_sx[r];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c = wn * 64 + 32 * i + 8 * g4 + 4 * fk;
                    const f32x4 sw = *reinterpret_cast<const f32x4*>(l_sw + c);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(l_b + c);
                    const int32_t a4[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                           acc[i][j][4 * g4 + 3]};
                    const u32x2 pk = epi_bf16x4(a4, sx, sw, bb, true);
                    const int off = r * 512 + (((c >> 3) ^ (r & 31)) << 4) + ((c & 7) << 1);
                    *reinterpret_cast<u32x2*>(smem + off) = pk;
                }
            }
        }
        __syncthreads();
        uint16_t* out = static_cast<uint16_t*>(ep.out);
        if (m0 + BM <= M && n0 + BN <= N) {
            // a whole tile: sixteen rows per instruction, a wave-uniform row base
            // plus a fixed 32-bit lane offset, no bounds checks
            const int c = tid & 31, rw = tid >> 5;
            const uint32_t o_lane = (uint32_t)(rw * ep.ldo + c * 8) * 2u;
            char* obase = reinterpret_cast<char*>(out + (int64_t)m0 * ep.ldo + n0);
#pragma unroll 4
            for (int it = 0; it < 16; ++it) {
                const int r = it * 16 + rw;
                const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * 512 + ((c ^ (r & 31)) << 4));
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (int64_t)it * 32 * ep.ldo + o_lane));
            }
        } else
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int q = it * NT8 + tid;
            const int r = q >> 5, c = q & 31;
            const int m = m0 + r;
            const int n = n0 + c * 8;
            if (m >= M || n >= N) continue;
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * 512 + ((c ^ (r & 31)) << 4));
            uint16_t* dst = out + (int64_t)m * ep.ldo + n;
            if (n + 7 < N) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));   // whole lines, streamed out
            } else {
                for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + wm * 128 + 32 * j + fr;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int n = n0 + wn * 64 + 32 * i + 8 * g4 + 4 * fk;
                    if (n >= N) continue;
                    const int32_t a4[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                           acc[i][j][4 * g4 + 3]};
                    store_i32x4(a4, n, N, m, ep);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wide kernel (K % 64 == 0, INT8 weights): a 256 x 384 output tile per
// workgroup of 8 waves, each wave 128 activation rows x 96 weight rows in
// twelve v_mfma_i32_32x32x32_i8 accumulators (192 registers).  Per MAC it
// moves 640 / (256 * 384) bytes from L2 into LDS instead of 512 / (256 * 256),
// 17 % less, which is what limits the 256 x 256 kernel (the copies' power
// and latency).  Same slice protocol as gemm_i8_w8_kernel with four 40 KB
// stages filling all 160 KB of LDS (activation copies of slice t+4 go into
// stage t after slice t's barrier, weight copies of slice t+3 at the start
// of slice t).  There is no room for a second set of activation fragments,
// so each activation fragment is reloaded with the next K half's data as soon
// as its three MFMAs are issued; the weight fragments are double-buffered.
// Epilogue: the scales and bias are loaded into registers once the last copy
// is issued (their latency hides under the last slices) and go to LDS above
// the staged rows after the K loop; the output tile is staged through the
// ring in four phases of 64 rows (768 bytes each, padded to 784) over two
// alternating 49 KB buffers, one barrier per phase, so one phase's stores
// overlap the next one's conversion; without bias it adds -0 (which changes
// no value) rather than selecting per output; whole tiles store through a wave-uniform row base plus fixed
// 32-bit lane offsets, with no per-store bounds checks or 64-bit addressing.
constexpr int BNW = 384;                        // weight rows per wide tile
constexpr int W12_NS = 4;
constexpr int W12_STG = (BM + BNW) * BK;        // 40 KB per stage
constexpr int W12_PER = 5;                      // copies per slice per thread (2 activation + 3 weight)

// staged output row: 768 bytes of BF16 plus 16 of padding, so that the 32
// rows written by a wave's lanes at one column start on 8 different 16-byte
// bank groups (rows 784 bytes apart) while every chunk stays 16-byte aligned
constexpr int W12_ROW = 784;

template <int MODE>
__global__ __launch_bounds__(NT8, 1) void gemm_i8_w12_kernel(const int8_t* __restrict__ A, int64_t lda, int64_t a_ss,
                                                            const int8_t* __restrict__ W, int64_t ldw, int64_t w_ss,
                                                            int M, int N, int K, EpiArgs ep) {
    constexpr int NS = W12_NS;
    constexpr int STG = W12_STG;
    constexpr int PER = W12_PER;
    constexpr int RING = NS * STG;                 // >= 128 rows x 768 bytes of staged output
    static_assert(RING >= 2 * 64 * W12_ROW + (BM + 2 * BNW) * 4, "output staging and epilogue operands");
    __shared__ __attribute__((aligned(1024))) int8_t smem[RING];
    float* l_sx = reinterpret_cast<float*>(smem + 2 * 64 * W12_ROW);   // after the K loop, above the staged rows
    float* l_sw = l_sx + 256;
    float* l_b = l_sw + BNW;

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BNW - 1) / BNW;
    const int T = tiles_m * tiles_n;
    const int g = blockIdx.x;
    const int xcd = g % NXCD;
    const int q8 = T / NXCD, rem = T % NXCD;
    const int t_lin = xcd * q8 + min(xcd, rem) + g / NXCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = t_lin / per_group;
    const int first_m = group * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tg = t_lin - group * per_group;
    const int m0 = (first_m + tg % gsz) * BM;
    const int n0 = (tg / gsz) * BNW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;    // 128-row half of the activation tile
    const int wn = wave >> 1;   // 96-row quarter of the weight tile

    // copy instruction i of this wave covers rows 16 * (wave + 8 i) + lane / 4
    // of the activation tile (i < 2) and of the weight tile (i < 3)
    // copy sources: tile base + slice offset (uniform) and a fixed per-lane offset
    uint32_t va[2], vw[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int rt = 16 * (wave + 8 * i) + (lane >> 2);
        const int c = (lane & 3) ^ swz(rt);
        if (i < 2) va[i] = (uint32_t)((int64_t)(min(m0 + rt, M - 1) - m0) * lda + c * 16);
        vw[i] = (uint32_t)((int64_t)(min(n0 + rt, N - 1) - n0) * ldw + c * 16);
    }
    const int8_t* a_base = A + (int64_t)m0 * lda;
    const int8_t* w_base = W + (int64_t)n0 * ldw;
    const uint32_t lds0 = lds_addr(smem);
    // slice u into LDS stage sg (= u % NS; a constant in the unrolled steady loop)
    auto copy_part = [&](int u, int sg, int part, int i) {
        const uint32_t sb = lds0 + (uint32_t)(sg * STG) + (uint32_t)(16 * (wave + 8 * i) * BK);
        if (part == 0) dma16s(sb, va[i], a_base + (int64_t)u * a_ss);
        else dma16s(sb + BM * BK, vw[i], w_base + (int64_t)u * w_ss);
    };

    // fragment b of a wave: rows base + 32 b + lane % 32, 16-byte chunk 2 kk + lane / 32;
    // the swizzle depends on bits 1 and 2 of the row only, i.e. on lane % 32
    const int fr = lane & 31;
    const int fk = lane >> 5;
    int a_off[2], w_off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        a_off[kk] = (wm * 128 + fr) * BK + (((2 * kk + fk) ^ swz(fr)) << 4);
        w_off[kk] = BM * BK + (wn * 96 + fr) * BK + (((2 * kk + fk) ^ swz(fr)) << 4);
    }
    auto rd_a = [&](int sg, int kk, int b) {
        return *reinterpret_cast<const i32x4*>(smem + sg * STG + a_off[kk] + b * 32 * BK);
    };
    auto rd_w = [&](int sg, int kk, int b) {
        return *reinterpret_cast<const i32x4*>(smem + sg * STG + w_off[kk] + b * 32 * BK);
    };

    i32x16 acc[3][4];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = K / BK;
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (u < nk) {
            copy_part(u, u, 0, 0);
            copy_part(u, u, 0, 1);
            copy_part(u, u, 1, 0);
            copy_part(u, u, 1, 1);
            copy_part(u, u, 1, 2);
        }
    wait_groups<PER>(min(nk, NS - 1) - 1);
    __syncthreads();   // slice 0 and the epilogue operands are visible
    if (NS - 1 < nk) {
        copy_part(NS - 1, NS - 1, 0, 0);
        copy_part(NS - 1, NS - 1, 0, 1);
    }

    // The loop runs from barrier to barrier (second half of slice t, then
    // first half of slice t + 1), so that no LDS read is pending at its back edge.
    i32x4 a[4], w0[3], w1[3];
    // STEADY: a slice with NS more after it, where every copy is issued and
    // two slices stay in flight (no run-time conditions in the loop body)
    // stage_tag: t % NS when the caller knows it at compile time, else -1
    auto first_half = [&](int t, auto steady_tag, auto stage_tag, auto extra_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int ST = decltype(stage_tag)::value;
        constexpr int XL = decltype(extra_tag)::value;   // loads issued after the last copy
        const int sc = ST >= 0 ? ST : t % NS;                              // slice t
        const int sp = ST >= 0 ? (ST + NS - 1) % NS : (t + NS - 1) % NS;   // slice t + NS - 1
        // first K half of slice t; its second half's fragments; weight copies of slice t+NS-1
        const bool late = STEADY || t + NS - 1 < nk;
        // raised priority while this half's MFMAs issue, normal again for the
        // barrier wait (measured: 0.6 % faster, same results)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < 3) w1[j] = rd_w(sc, 1, j);
#pragma unroll
            for (int i = 0; i < 3; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w0[i], a[j], acc[i][j], 0, 0, 0);
            a[j] = rd_a(sc, 1, j);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (late && j < 3) copy_part(t + NS - 1, sp, 1, j);
            __builtin_amdgcn_sched_barrier(0);
        }
        acc[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[0], a[0], acc[0][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (STEADY) wait_vmcnt<(NS - 2) * PER>();
        else wait_groups_x<PER, XL>(min(nk - 1, t + NS - 1) - (t + 1));
        __builtin_amdgcn_s_barrier();
    };
    auto second_half = [&](int t, bool next, auto steady_tag, auto stage_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int ST = decltype(stage_tag)::value;
        const int sc = ST >= 0 ? ST : t % NS;                   // slice t (and t + NS)
        const int sn = ST >= 0 ? (ST + 1) % NS : (t + 1) % NS;  // slice t + 1
        // second K half of slice t; slice t+1's first-half fragments; activation copies of slice t+NS
        const bool early = STEADY || t + NS < nk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (next && j < 3) w0[j] = rd_w(sn, 0, j);
#pragma unroll
            for (int i = 0; i < 3; ++i)
                if (i != 0 || j != 0)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w1[i], a[j], acc[i][j], 0, 0, 0);
            if (next) a[j] = rd_a(sn, 0, j);
            if (j == 0) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (early && j < 2) copy_part(t + NS, sc, 0, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
#pragma unroll
    for (int b = 0; b < 4; ++b) a[b] = rd_a(0, 0, b);
#pragma unroll
    for (int b = 0; b < 3; ++b) w0[b] = rd_w(0, 0, b);
    using rt = std::integral_constant<int, -1>;
    using x0 = std::integral_constant<int, 0>;
    first_half(0, std::false_type{}, std::integral_constant<int, 0>{}, x0{});
    // steady slices NS at a time, so that each one's LDS stages are constants
    static_assert(NS == 4, "the unrolled steady loop covers four stages");
    auto steady = [&](int t0, auto jt) {
        constexpr int J = decltype(jt)::value;
        second_half(t0 + J, true, std::true_type{}, std::integral_constant<int, J>{});
        first_half(t0 + J + 1, std::true_type{}, std::integral_constant<int, (J + 1) % NS>{}, x0{});
    };
    int t = 0;
    for (; t + 2 * NS - 1 < nk; t += NS) {
        steady(t, std::integral_constant<int, 0>{});
        steady(t, std::integral_constant<int, 1>{});
        steady(t, std::integral_constant<int, 2>{});
        steady(t, std::integral_constant<int, 3>{});
    }
    for (; t + NS < nk; ++t) {
        second_half(t, true, std::true_type{}, rt{});
        first_half(t + 1, std::true_type{}, rt{}, x0{});
    }
    // Every copy is issued now.  The epilogue's scales and bias are loaded here,
    // three loads in every lane, so that the last slices hide their latency; the
    // waits below allow those three loads to remain in flight.
    constexpr int XL = MODE == MODE_BF16 ? 3 : 0;
    float e_sx = 0.0f, e_sw = 0.0f;
    uint16_t e_b = 0;
    if constexpr (MODE == MODE_BF16) {
        // the thread index rebuilt from the lane count (the compiler keeps
        // threadIdx spilled across the K loop, and its reload would make it wait
        // for the copies still in flight)
        const int lt = wave * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int n = min(n0 + lt % BNW, N - 1);
        e_sx = ep.a_scale[min(m0 + (lt & (BM - 1)), M - 1) * ep.a_step];
        e_sw = ep.w_scale[n * ep.w_step];
        e_b = *(ep.bias ? ep.bias + n : reinterpret_cast<const uint16_t*>(ep.w_scale));
    }
    for (; t + 1 < nk; ++t) {
        second_half(t, true, std::false_type{}, rt{});
        first_half(t + 1, std::false_type{}, rt{}, std::integral_constant<int, XL>{});
    }
    second_half(nk - 1, false, std::false_type{}, rt{});

    if (MODE == MODE_BF16) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();   // the ring is free
        if (tid < BM) l_sx[tid] = e_sx;
        if (tid < BNW) {
            l_sw[tid] = e_sw;
            // without bias, -0: adding it changes no value (unlike +0, which turns -0 into +0)
            l_b[tid] = ep.bias ? bf16_to_f32(e_b) : -0.0f;
        }
        // Four phases, one 32-row fragment j = ph of every wave each: tile rows
        // wm * 128 + 32 ph + lane % 32 -> staged row wm * 32 + lane % 32 of a
        // 64-row (48 KB) buffer; the two buffers alternate, so one barrier per
        // phase keeps every buffer written before it is read and read before it
        // is rewritten, and a phase's stores overlap the next phase's conversion.
        // Thread chunk it of a phase: staged row q / 48, 16-byte chunk q % 48
        // (q = it * 512 + tid); its offsets are the same in every phase.
        uint32_t o_off[6], l_off[6];
#pragma unroll
        for (int it = 0; it < 6; ++it) {
            const int q = it * NT8 + tid;
            const int sr = q / 48, ch = q - 48 * (q / 48);
            const int tr = (sr >> 5) * 128 + (sr & 31);   // tile row in phase 0
            o_off[it] = (uint32_t)(tr * ep.ldo + ch * 8) * 2u;
            l_off[it] = (uint32_t)(sr * W12_ROW + ch * 16);
        }
        const bool full = m0 + BM <= M && n0 + BNW <= N;
        __syncthreads();
        char* out = static_cast<char*>(ep.out);
#pragma unroll
        for (int ph = 0; ph < 4; ++ph) {
            int8_t* buf = smem + (ph & 1) * (64 * W12_ROW);
            const float sx = l_sx[wm * 128 + 32 * ph + fr];
            const int sr = wm * 32 + fr;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c = wn * 96 + 32 * i + 8 * g4 + 4 * fk;
                    const f32x4 sw = *reinterpret_cast<const f32x4*>(l_sw + c);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(l_b + c);
                    const int32_t a4[4] = {acc[i][ph][4 * g4], acc[i][ph][4 * g4 + 1], acc[i][ph][4 * g4 + 2],
                                           acc[i][ph][4 * g4 + 3]};
                    const u32x2 pk = epi_bf16x4(a4, sx, sw, bb, true);
                    *reinterpret_cast<u32x2*>(buf + sr * W12_ROW + 2 * c) = pk;
                }
            }
            __syncthreads();
            char* obase = out + ((int64_t)(m0 + 32 * ph) * ep.ldo + n0) * 2;   // the phase's first output row
            if (full) {
#pragma unroll
                for (int it = 0; it < 6; ++it) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + l_off[it]);
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + o_off[it]));
                }
            } else {
#pragma unroll
                for (int it = 0; it < 6; ++it) {
                    const int q = it * NT8 + tid;
                    const int sr2 = q / 48, ch = q - 48 * (q / 48);
                    const int m = m0 + (sr2 >> 5) * 128 + 32 * ph + (sr2 & 31);
                    const int n = n0 + ch * 8;
                    if (m >= M || n >= N) continue;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + l_off[it]);
                    uint16_t* dst = reinterpret_cast<uint16_t*>(obase + o_off[it]);
                    if (n + 7 < N) {
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
                    } else {
                        for (int e = 0; e < 8 && n + e < N; ++e)
                            dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + wm * 128 + 32 * j + fr;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int n = n0 + wn * 96 + 32 * i + 8 * g4 + 4 * fk;
                    if (n >= N) continue;
                    const int32_t a4[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                           acc[i][j][4 * g4 + 3]};
                    store_i32x4(a4, n, N, m, ep);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// FP6 operands (W4A4 codes on the FP6 matrix path).  Every INT4 code in
// [-7, 7] is exact in FP6 E2M3, and v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit (E8M0 = 127) scales multiplies 32 x 64 by 64 x 32 FP6 blocks at twice
// the INT8 rate, accumulating in FP32.  All partial sums are integers of
// magnitude <= K * 49 < 2^24, so the FP32 accumulator holds the exact INT32
// sum and the epilogue sees the same value as the INT8 path.
//
// The loop is the eight-wave INT8 kernel's protocol (barrier between the two
// K halves of a slice) with a slice of 128 values: 96 bytes per row, one
// MFMA K step (64 values, 48 bytes) per half.  Operands arrive in the FP6
// operand format (qdiff.h): per 64-value block, [piece 0 bytes 0..15 |
// piece 1 bytes 0..15 | tails], the tails swapped when bits 3 and 4 of the
// row differ.  In LDS a row's slice is six 16-byte slots (96 bytes, so one
// copy instruction moves ~11 whole row slices), with the two K steps' slot
// groups exchanged when bits 2 and 3 of the row differ.  A lane (row r, K
// half h) takes piece h as one 16-byte read (its head slot) and one 8-byte
// read (tail half h ^ swap(r)).  The exchange and the swap together put the
// rows of every read phase on distinct banks (for 32 or 64 banks), so both
// reads are free of bank conflicts.  Three 48 KB stages.
constexpr int F6_BK = 128;                 // values per slice
constexpr int F6_RB = 96;                  // bytes per row per slice
constexpr int F6_STG = (BM + BN) * F6_RB;  // 48 KB per stage
constexpr int F6_NS = 3;

__device__ __forceinline__ int f6_rot(int r) { return 3 * (((r >> 2) ^ (r >> 3)) & 1); }   // slots
__device__ __forceinline__ int f6_swp(int r) { return ((r >> 3) ^ (r >> 4)) & 1; }

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four outputs from exact FP32 sums (same arithmetic as epi_bf16x4).
__device__ __forceinline__ u32x2 epi_bf16x4_f(const float* a4, float sx, const f32x4& sw, const f32x4& b,
                                              bool has_bias) {
#pragma clang fp contract(off)
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float tt = a4[e];
        tt = tt * sx;
        tt = tt * sw[e];
        if (has_bias) tt = tt + b[e];
        o[e] = tt;
    }
    u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    return pk;
}

// ---------------------------------------------------------------------------
// The FP6 kernel: a 256 x 256 tile computed by four waves (one per SIMD),
// each 128 x 128 in sixteen accumulators held in the accumulator registers,
// so that every fragment read from LDS feeds four MFMAs (eight waves of
// 128 x 64 need a third more LDS reads per MFMA and ran 2-7 % slower).  The
// MFMA operands are 6-register FP6 tuples (the intrinsic's 6-dword form),
// two registers fewer per fragment than the 8-dword builtin.
typedef int32_t i32x6 __attribute__((ext_vector_type(6)));
}  // namespace
// (declared outside the unnamed namespace: the asm label binds it to the
// compiler's intrinsic, so it has no definition of its own)
__device__ f32x16 mfma_f6x6(i32x6 a, i32x6 b, f32x16 c, int cbsz, int blgp, int opsel_a, int scale_a, int opsel_b,
                            int scale_b) __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v6i32.v6i32");
namespace {

constexpr int NT4 = 256;
constexpr int F6W4_PER = 12;   // copies per slice per thread (6 activation + 6 weight)

template <int MODE>
__global__ __launch_bounds__(NT4, 1) void gemm_f6_w4_kernel(const uint8_t* __restrict__ A, int64_t lda, int64_t a_ss,
                                                           const uint8_t* __restrict__ W, int64_t ldw, int64_t w_ss,
                                                           int M, int N, int K, EpiArgs ep) {
    constexpr int NS = F6_NS;
    constexpr int STG = F6_STG;
    constexpr int PER = F6W4_PER;
    constexpr int RING = NS * STG > 256 * 512 ? NS * STG : 256 * 512;
    __shared__ __attribute__((aligned(1024))) int8_t smem[RING + EPI_LDS];
    float* l_sx = reinterpret_cast<float*>(smem + RING);
    float* l_sw = l_sx + 256;
    float* l_b = l_sw + 256;

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int T = tiles_m * tiles_n;
    const int g = blockIdx.x;
    const int xcd = g % NXCD;
    const int q8 = T / NXCD, rem = T % NXCD;
    const int t_lin = xcd * q8 + min(xcd, rem) + g / NXCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = t_lin / per_group;
    const int first_m = group * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tg = t_lin - group * per_group;
    const int m0 = (first_m + tg % gsz) * BM;
    const int n0 = (tg / gsz) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;    // 128-row half of the activation tile
    const int wn = wave >> 1;   // 128-row half of the weight tile

    if (MODE == MODE_BF16) {
        l_sx[tid] = ep.a_scale[min(m0 + tid, M - 1) * ep.a_step];
        const int n = min(n0 + tid, N - 1);
        l_sw[tid] = ep.w_scale[n * ep.w_step];
        // without bias, -0: adding it changes no value (unlike +0, which turns -0 into +0)
        l_b[tid] = ep.bias ? bf16_to_f32(ep.bias[n]) : -0.0f;
    }

    // copies: instruction i (0..5) of wave w fills the 16-byte LDS slots
    // (6w + i) * 64 + lane of an operand's 24 KB stage part (slot layout
    // above: six slots per row slice, rotated by f6_rot(row))
    uint32_t va[6], vw[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int q = (6 * wave + i) * 64 + lane;
        const int row = q / 6;
        const int phys = q - 6 * row;
        const int logical = (phys + f6_rot(row)) % 6;
        va[i] = (uint32_t)((int64_t)(min(m0 + row, M - 1) - m0) * lda + 16 * logical);
        vw[i] = (uint32_t)((int64_t)(min(n0 + row, N - 1) - n0) * ldw + 16 * logical);
    }
    const int8_t* a_base = reinterpret_cast<const int8_t*>(A) + (int64_t)m0 * lda;
    const int8_t* w_base = reinterpret_cast<const int8_t*>(W) + (int64_t)n0 * ldw;
    const uint32_t lds0 = lds_addr(smem);
    // slice u into LDS stage sg (= u % NS, a constant in the unrolled steady loop)
    auto copy_part = [&](int u, int sg, int part, int i) {
        const uint32_t sb = lds0 + (uint32_t)(sg * STG) + (uint32_t)((6 * wave + i) * 1024);
        if (part == 0) dma16s(sb, va[i], a_base + (int64_t)u * a_ss);
        else dma16s(sb + BM * F6_RB, vw[i], w_base + (int64_t)u * w_ss);
    };

    const int fr = lane & 31;
    const int fk = lane >> 5;
    // fragment b covers rows base + 32 b + lane % 32; the slot rotation and tail
    // swap depend on row bits 2..4 only, i.e. on lane % 32, so all b share them
    const int ra = wm * 128 + fr, rw = wn * 128 + fr;
    int a_h[2], a_t[2], w_h[2], w_t[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        a_h[kk] = ra * F6_RB + 16 * ((3 * kk + fk + f6_rot(ra)) % 6);
        a_t[kk] = ra * F6_RB + 16 * ((3 * kk + 2 + f6_rot(ra)) % 6) + 8 * (fk ^ f6_swp(ra));
        w_h[kk] = BM * F6_RB + rw * F6_RB + 16 * ((3 * kk + fk + f6_rot(rw)) % 6);
        w_t[kk] = BM * F6_RB + rw * F6_RB + 16 * ((3 * kk + 2 + f6_rot(rw)) % 6) + 8 * (fk ^ f6_swp(rw));
    }
    auto rd = [&](int sg, int head, int tail, int b) {
        const int8_t* base = smem + sg * STG + b * 32 * F6_RB;
        const i32x4 h = *reinterpret_cast<const i32x4*>(base + head);
        const u32x2 t = *reinterpret_cast<const u32x2*>(base + tail);
        return i32x6{h[0], h[1], h[2], h[3], (int32_t)t[0], (int32_t)t[1]};
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / F6_BK;
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (u < nk) {
#pragma unroll
            for (int i = 0; i < 6; ++i) copy_part(u, u, 0, i);
#pragma unroll
            for (int i = 0; i < 6; ++i) copy_part(u, u, 1, i);
        }
    wait_groups<PER>(min(nk, NS - 1) - 1);
    __syncthreads();
    if (NS - 1 < nk) {
#pragma unroll
        for (int i = 0; i < 6; ++i) copy_part(NS - 1, NS - 1, 0, i);
    }

    i32x6 a0[4], w0[4], a1[4], w1[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        a0[b] = rd(0, a_h[0], a_t[0], b);
        w0[b] = rd(0, w_h[0], w_t[0], b);
    }
    // STEADY: a slice with NS more after it (every copy issued, one slice in flight)
    auto slice = [&](int t, auto steady_tag, auto stage_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        constexpr int ST = decltype(stage_tag)::value;   // t % NS when known, else -1
        const int sc = ST >= 0 ? ST : t % NS;
        const int sn = ST >= 0 ? (ST + 1) % NS : (sc + 1 == NS ? 0 : sc + 1);
        const int sp = ST >= 0 ? (ST + NS - 1) % NS : (sc == 0 ? NS - 1 : sc - 1);
        const bool late = STEADY || t + NS - 1 < nk;
        // first K step of slice t; reads of its second step; weight copies of slice t+NS-1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w1[q] = rd(sc, w_h[1], w_t[1], q);
            a1[q] = rd(sc, a_h[1], a_t[1], q);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[q][j] = mfma_f6x6(w0[q], a0[j], acc[q][j], 2, 2, 0, 127, 0, 127);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (late) {
                if (q == 0) { copy_part(t + NS - 1, sp, 1, 0); copy_part(t + NS - 1, sp, 1, 1); }
                if (q == 1) copy_part(t + NS - 1, sp, 1, 2);
                if (q == 2) { copy_part(t + NS - 1, sp, 1, 3); copy_part(t + NS - 1, sp, 1, 4); }
                if (q == 3) copy_part(t + NS - 1, sp, 1, 5);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        acc[0][0] = mfma_f6x6(w1[0], a1[0], acc[0][0], 2, 2, 0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (STEADY) wait_vmcnt<(NS - 2) * PER>();
        else wait_groups<PER>(min(nk - 1, t + NS - 1) - (t + 1));
        __builtin_amdgcn_s_barrier();
        const bool early = STEADY || t + NS < nk;
        // second K step of slice t; reads of slice t+1's first step; activation copies of slice t+NS
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0[q] = rd(sn, w_h[0], w_t[0], q);
            a0[q] = rd(sn, a_h[0], a_t[0], q);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (q != 0 || j != 0) acc[q][j] = mfma_f6x6(w1[q], a1[j], acc[q][j], 2, 2, 0, 127, 0, 127);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (early) {
                if (q == 0) { copy_part(t + NS, sc, 0, 0); copy_part(t + NS, sc, 0, 1); }
                if (q == 1) copy_part(t + NS, sc, 0, 2);
                if (q == 2) { copy_part(t + NS, sc, 0, 3); copy_part(t + NS, sc, 0, 4); }
                if (q == 3) copy_part(t + NS, sc, 0, 5);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // steady slices three at a time, so that each one's LDS stages are
    // constants (with three stages, t % NS would otherwise cost a division
    // and a dozen address adds per slice), then the rest
    static_assert(NS == 3, "the unrolled steady loop assumes three stages");
    int t = 0;
    for (; t + NS + 2 < nk; t += 3) {
        slice(t, std::true_type{}, std::integral_constant<int, 0>{});
        slice(t + 1, std::true_type{}, std::integral_constant<int, 1>{});
        slice(t + 2, std::true_type{}, std::integral_constant<int, 2>{});
    }
    for (; t + NS < nk; ++t) slice(t, std::true_type{}, std::integral_constant<int, -1>{});
    for (; t < nk; ++t) slice(t, std::false_type{}, std::integral_constant<int, -1>{});

    if (MODE == MODE_BF16) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        // acc[i][j][4 g4 + e]: (n, m) = (wn*128 + 32 i + 8 g4 + 4 fk + e, wm*128 + 32 j + fr) in the tile
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wm * 128 + 32 * j + fr;
            const float sx = l_sx[r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c = wn * 128 + 32 * i + 8 * g4 + 4 * fk;
                    const f32x4 sw = *reinterpret_cast<const f32x4*>(l_sw + c);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(l_b + c);
                    const float a4[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                         acc[i][j][4 * g4 + 3]};
                    const u32x2 pk = epi_bf16x4_f(a4, sx, sw, bb, true);
                    const int off = r * 512 + (((c >> 3) ^ (r & 31)) << 4) + ((c & 7) << 1);
                    *reinterpret_cast<u32x2*>(smem + off) = pk;
                }
            }
        }
        __syncthreads();
        uint16_t* out = static_cast<uint16_t*>(ep.out);
        if (m0 + BM <= M && n0 + BN <= N) {
            // a whole tile: eight rows per instruction, a wave-uniform row base
            // plus a fixed 32-bit lane offset, no bounds checks
            const int c = tid & 31, rw = tid >> 5;
            const uint32_t o_lane = (uint32_t)(rw * ep.ldo + c * 8) * 2u;
            char* obase = reinterpret_cast<char*>(out + (int64_t)m0 * ep.ldo + n0);
#pragma unroll 4
            for (int it = 0; it < 32; ++it) {
                const int r = it * 8 + rw;
                const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * 512 + ((c ^ (r & 31)) << 4));
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (int64_t)it * 16 * ep.ldo + o_lane));
            }
        } else
#pragma unroll 4
        for (int it = 0; it < 32; ++it) {
            const int q = it * NT4 + tid;
            const int r = q >> 5, c = q & 31;
            const int m = m0 + r;
            const int n = n0 + c * 8;
            if (m >= M || n >= N) continue;
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * 512 + ((c ^ (r & 31)) << 4));
            uint16_t* dst = out + (int64_t)m * ep.ldo + n;
            if (n + 7 < N) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
            } else {
                for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + wm * 128 + 32 * j + fr;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int n = n0 + wn * 128 + 32 * i + 8 * g4 + 4 * fk;
                    if (n >= N) continue;
                    const int32_t a4[4] = {(int32_t)acc[i][j][4 * g4], (int32_t)acc[i][j][4 * g4 + 1],
                                           (int32_t)acc[i][j][4 * g4 + 2], (int32_t)acc[i][j][4 * g4 + 3]};
                    store_i32x4(a4, n, N, m, ep);
                }
            }
        }
    }
}

// Operand addressing: row-major (row n at wq + n * ldw), or K-sliced (byte
// (n, k) at (k / 64) * N * 64 + n * 64 + k % 64, K % 64 == 0): the 64-byte
// K slices of consecutive rows are adjacent, so each copy instruction of
// the eight-wave kernels reads 1 KB of consecutive bytes (eight whole
// 128-byte lines instead of sixteen half lines).  Either operand may be
// K-sliced (the weights offline, the activation codes by the quantizer).
template <int MODE>
hipError_t launch(const int8_t* aq, int64_t lda, const int8_t* wq, int64_t ldw, bool w_sliced, bool a_sliced,
                  int64_t M, int64_t N, int64_t K, const EpiArgs& ep, hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t w_rs = w_sliced ? BK : ldw;
    const int64_t w_ss = w_sliced ? N * BK : BK;
    const int64_t a_rs = a_sliced ? BK : lda;
    const int64_t a_ss = a_sliced ? M * BK : BK;
    if (gemm_uses_wide_tiles(M, N, K))
        gemm_i8_w12_kernel<MODE><<<dim3((unsigned)(((M + BM - 1) / BM) * ((N + BNW - 1) / BNW))), dim3(NT8), 0,
                                   stream>>>(aq, a_rs, a_ss, wq, w_rs, w_ss, (int)M, (int)N, (int)K, ep);
    else if (K % BK == 0)
        gemm_i8_w8_kernel<MODE, 4, WF_I8><<<dim3((unsigned)tiles), dim3(NT8), 0, stream>>>(
            aq, a_rs, a_ss, wq, w_rs, w_ss, (int)M, (int)N, (int)K, ep);
    else if (!w_sliced && !a_sliced)
        gemm_i8_kernel<MODE><<<dim3((unsigned)tiles), dim3(NT), 0, stream>>>(aq, lda, wq, ldw, (int)M,
                                                                            (int)N, (int)K, ep);
    else
        return hipErrorInvalidValue;   // K-sliced weights need K % 64 == 0 (checked by the callers)
    return hipGetLastError();
}

// 16-byte chunk o of a K-sliced copy with slices of SB bytes per row:
// slice o / (R * SB / 16), row (o / (SB / 16)) % R, piece o % (SB / 16).
template <int SB>
__global__ __launch_bounds__(256) void slice_rows_kernel(const uint8_t* __restrict__ src, int64_t ld, int64_t R,
                                                         int64_t chunks, uint8_t* __restrict__ out) {
    constexpr int CPR = SB / 16;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < chunks; o += (int64_t)gridDim.x * 256) {
        const int64_t u = o / (CPR * R);
        const int64_t r = o - u * CPR * R;
        const int64_t row = r / CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + row * ld + u * SB + (r - row * CPR) * 16);
        *reinterpret_cast<u32x4*>(out + o * 16) = v;
    }
}

template <int SB>
hipError_t launch_slice_rows(const uint8_t* src, int64_t ld, int64_t R, int64_t nslices, uint8_t* out,
                             hipStream_t stream) {
    const int64_t chunks = nslices * R * (SB / 16);
    const int64_t blocks = (chunks + 255) / 256 < 65536 ? (chunks + 255) / 256 : 65536;
    slice_rows_kernel<SB><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(src, ld, R, chunks, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const int8_t* aq, int64_t lda, const float* a_scale, const int8_t* wq,
                            int64_t ldw, const float* w_scale, const void* bias, void* y,
                            int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                            int a_step, int w_step, bool w_sliced, bool a_sliced) {
    EpiArgs ep{a_scale, w_scale, static_cast<const uint16_t*>(bias), y, ldy, a_step, w_step};
    return launch<MODE_BF16>(aq, lda, wq, ldw, w_sliced, a_sliced, M, N, K, ep, stream);
}

hipError_t launch_gemm_i32(const int8_t* aq, int64_t lda, const int8_t* wq, int64_t ldw,
                           int32_t* acc, int64_t ldc, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream, bool w_sliced, bool a_sliced) {
    EpiArgs ep{nullptr, nullptr, nullptr, acc, ldc, 0, 0};
    return launch<MODE_I32>(aq, lda, wq, ldw, w_sliced, a_sliced, M, N, K, ep, stream);
}

hipError_t launch_slice_weights(const int8_t* wq, int64_t ldw, int64_t N, int64_t K, int8_t* out,
                                hipStream_t stream) {
    return launch_slice_rows<BK>(reinterpret_cast<const uint8_t*>(wq), ldw, N, K / BK, reinterpret_cast<uint8_t*>(out),
                                 stream);
}

hipError_t launch_slice_fp6(const uint8_t* w6, int64_t ldw, int64_t N, int64_t K, uint8_t* out, hipStream_t stream) {
    return launch_slice_rows<F6_RB>(w6, ldw, N, K / F6_BK, out, stream);
}

// Packed-INT4 weights (K % 64 == 0): five 24 KB stages, four slices in flight.
hipError_t launch_gemm_w4_bf16(const int8_t* aq, int64_t lda, const float* a_scale, const uint8_t* wp,
                               int64_t ldw, const float* w_scale, const void* bias, void* y,
                               int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                               int a_step, int w_step) {
    EpiArgs ep{a_scale, w_scale, static_cast<const uint16_t*>(bias), y, ldy, a_step, w_step};
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_i8_w8_kernel<MODE_BF16, 5, WF_I4><<<dim3((unsigned)tiles), dim3(NT8), 0, stream>>>(
        aq, lda, BK, reinterpret_cast<const int8_t*>(wp), ldw, BK / 2, (int)M, (int)N, (int)K, ep);
    return hipGetLastError();
}

// FP6 operands row-major (row stride ld bytes) or K-sliced (96-byte slices,
// byte (r, b) at (b / 96) * R * 96 + r * 96 + b % 96).
hipError_t launch_gemm_f6_bf16(const uint8_t* a6, int64_t lda, const float* a_scale, const uint8_t* w6,
                               int64_t ldw, const float* w_scale, const void* bias, void* y, int64_t ldy,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream, bool w_sliced, bool a_sliced) {
    EpiArgs ep{a_scale, w_scale, static_cast<const uint16_t*>(bias), y, ldy, 1, 1};
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_f6_w4_kernel<MODE_BF16><<<dim3((unsigned)tiles), dim3(NT4), 0, stream>>>(
        a6, a_sliced ? F6_RB : lda, a_sliced ? M * F6_RB : F6_RB, w6, w_sliced ? F6_RB : ldw,
        w_sliced ? N * F6_RB : F6_RB, (int)M, (int)N, (int)K, ep);
    return hipGetLastError();
}

hipError_t launch_gemm_f6_i32(const uint8_t* a6, int64_t lda, const uint8_t* w6, int64_t ldw, int32_t* acc,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, hipStream_t stream, bool w_sliced,
                              bool a_sliced) {
    EpiArgs ep{nullptr, nullptr, nullptr, acc, ldc, 0, 0};
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_f6_w4_kernel<MODE_I32><<<dim3((unsigned)tiles), dim3(NT4), 0, stream>>>(
        a6, a_sliced ? F6_RB : lda, a_sliced ? M * F6_RB : F6_RB, w6, w_sliced ? F6_RB : ldw,
        w_sliced ? N * F6_RB : F6_RB, (int)M, (int)N, (int)K, ep);
    return hipGetLastError();
}

hipError_t launch_gemm_w4_i32(const int8_t* aq, int64_t lda, const uint8_t* wp, int64_t ldw,
                              int32_t* acc, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
    EpiArgs ep{nullptr, nullptr, nullptr, acc, ldc, 0, 0};
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_i8_w8_kernel<MODE_I32, 5, WF_I4><<<dim3((unsigned)tiles), dim3(NT8), 0, stream>>>(
        aq, lda, BK, reinterpret_cast<const int8_t*>(wp), ldw, BK / 2, (int)M, (int)N, (int)K, ep);
    return hipGetLastError();
}

}  // namespace qd
