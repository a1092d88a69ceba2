// Measurement kernels for the benchmark (not part of the layer's path):
//  * the achievable dense INT8 matrix-core rate on this machine, with
//    operands that change from one v_mfma_i32_32x32x32_i8 to the next (the
//    power, and so the clock, depends on the data the matrix cores see);
//  * HBM streaming bandwidth for three read/write mixes (read only, copy,
//    and two bytes read per byte written, the quantizer's mix);
//  * a clock sample (shader cycle counter and constant-rate wall counter,
//    per workgroup with its XCD) for the average shader clock between two
//    points of a stream.
// Built into its own library (libqdmeasure.so); every entry point is
// extern "C" and returns the launch status (0 = success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Each wave holds eight random A and eight random B fragments and runs eight
// independent accumulator chains, rotating the operand pair on every MFMA:
// 64 MFMAs (64 x 65536 INT8 operations) per wave per iteration.
__global__ __launch_bounds__(kThreads, 2) void mfma_i8_kernel(const i32x4* __restrict__ src, int64_t mask,
                                                              int iters, int32_t* __restrict__ sink) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    i32x4 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = src[(t * 16 + i) & mask];
        b[i] = src[(t * 16 + 8 + i) & mask];
    }
    i32x16 acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[q][e] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(r + q) & 7], b[(3 * r + q) & 7], acc[q], 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) s ^= acc[q][e];
    if (s == 0x13572468) sink[t & 1023] = s;   // keeps the work; practically never stored
}

// Streaming kernels over n 16-byte chunks with non-temporal accesses, several
// chunks per thread in flight (eight for reads, four for copies, two output
// chunks for the 2:1 mix).
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ a, int64_t n,
                                                        int32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t s = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = i + u * stride < n ? __builtin_nontemporal_load(a + i + u * stride) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 8; ++u) s ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (s == 0x13572468u) sink[threadIdx.x] = (int32_t)s;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b,
                                                        int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * stride < n) v[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * stride < n) __builtin_nontemporal_store(v[u], b + i + u * stride);
    }
}

// n output chunks: out[i] = a[2i] ^ a[2i + 1] (32 bytes read per 16 written).
__global__ __launch_bounds__(kThreads) void mix21_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b,
                                                         int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += 2 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (i + u * stride < n) {
                v[2 * u] = __builtin_nontemporal_load(a + 2 * (i + u * stride));
                v[2 * u + 1] = __builtin_nontemporal_load(a + 2 * (i + u * stride) + 1);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (i + u * stride < n) __builtin_nontemporal_store(v[2 * u] ^ v[2 * u + 1], b + i + u * stride);
    }
}

// Per workgroup: shader cycle counter, constant-rate wall counter, XCD and
// hardware id (compute unit, shader array and engine).  The cycle counters of
// different compute units are not aligned with one another, so two samples
// are only compared on the same compute unit.
__global__ void clock_kernel(uint64_t* __restrict__ out) {
    if (threadIdx.x == 0) {
        const uint64_t c = __builtin_readcyclecounter();
        const uint64_t w = (uint64_t)wall_clock64();
        // HW_REG_XCC_ID (hardware register 20), bits 3..0: the XCD of this wave
        const uint32_t xcc = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11));
        // HW_REG_HW_ID (hardware register 4), all 32 bits
        const uint32_t hw = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));
        out[4 * blockIdx.x + 0] = c;
        out[4 * blockIdx.x + 1] = w;
        out[4 * blockIdx.x + 2] = xcc & 0xFu;
        out[4 * blockIdx.x + 3] = hw;
    }
}

}  // namespace

extern "C" {

// src: random 16-byte vectors, a power-of-two count (mask + 1); blocks of 256
// threads (two fit a CU); sink: >= 1024 int32.  Operations per launch:
// blocks * 4 waves * iters * 64 * 65536.
int qdm_mfma_i8(const void* src, int64_t vecs, int blocks, int iters, int32_t* sink, hipStream_t stream) {
    if (vecs <= 0 || (vecs & (vecs - 1)) != 0 || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    mfma_i8_kernel<<<blocks, kThreads, 0, stream>>>(static_cast<const i32x4*>(src), vecs - 1, iters, sink);
    return (int)hipGetLastError();
}

// Bytes must be a multiple of 16 (of 32 for mix21's input); sink >= 256 int32.
int qdm_read(const void* a, int64_t bytes, int blocks, int32_t* sink, hipStream_t stream) {
    if (bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    read_kernel<<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(a), bytes / 16, sink);
    return (int)hipGetLastError();
}

int qdm_copy(const void* a, void* b, int64_t bytes, int blocks, hipStream_t stream) {
    if (bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    copy_kernel<<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(a), static_cast<u32x4*>(b), bytes / 16);
    return (int)hipGetLastError();
}

// Reads 2 * out_bytes from a, writes out_bytes to b.
int qdm_mix21(const void* a, void* b, int64_t out_bytes, int blocks, hipStream_t stream) {
    if (out_bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    mix21_kernel<<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(a), static_cast<u32x4*>(b),
                                                  out_bytes / 16);
    return (int)hipGetLastError();
}

// out: 4 * blocks uint64 (cycle counter, wall counter, XCD, hardware id per workgroup).
int qdm_clock_sample(uint64_t* out, int blocks, hipStream_t stream) {
    if (blocks <= 0) return (int)hipErrorInvalidValue;
    clock_kernel<<<blocks, 64, 0, stream>>>(out);
    return (int)hipGetLastError();
}

// Rate of the wall counter in kHz (device 0 of the calling thread's view).
int qdm_wall_clock_khz(void) {
    int dev = 0, r = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return r;
}

}  // extern "C"
