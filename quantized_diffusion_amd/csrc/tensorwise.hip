// Tensor-wise INT8 quantization for gfx950 (CDNA4).
//
// quantize_int8_tensorwise (comfy-kitchen 0.2.40 page, "Huawei Ascend
// backend"): one scale for the whole M x K tensor, s = amax / 127 where amax
// is the largest |x| over every element, and codes clamp(rne(fl(x / s))),
// all zero when s == 0.  No rotation.
//
// Two launches on the caller's stream, no atomics and no memset:
//  1. tw_amax_kernel: workgroup g takes rows g, g + G, ... and writes the
//     largest |x| it saw to partial[g] (the caller's workspace);
//  2. tw_quant_kernel: every workgroup reduces partial[0 .. G) (a maximum is
//     exact in any order), forms s and r = fl(1/s), and quantizes rows
//     M-1-g, M-1-g-G, ... with the reciprocal fast path and the
//     exact-division fallback of the per-row quantizer; workgroup 0 writes s.
// Each thread keeps U 16-byte chunks of a row in flight per iteration.
// The second pass walks the rows in the opposite order to the first: the
// rows the first pass read last are the ones most likely still held in the
// memory-side cache (256 MB on MI355X, smaller than a large activation), so
// they are read first, before the pass's own reads evict them.  The codes
// are stored with the streaming hint so that they do not evict those rows
// either (a GEMM reading the codes right after measured no slower for it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qd_device.h"
#include "qd_launch.h"
#include "qd_quant.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int U = 4;            // chunks per thread per row pass

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = __builtin_fmaxf(m, red[i]);
    return m;
}

template <class In>
__global__ __launch_bounds__(kThreads) void tw_amax_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                           int M, int cpr, float* __restrict__ partial) {
    constexpr int E = In::E;
    __shared__ float red[kThreads / 64];
    float am = 0.0f;
    for (int row = blockIdx.x; row < M; row += gridDim.x) {
        const uint8_t* src = x + (int64_t)row * ldx_bytes;
        for (int c0 = 0; c0 < cpr; c0 += U * kThreads) {
            u32x4 d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kThreads + (int)threadIdx.x;
                d[u] = c < cpr ? *reinterpret_cast<const u32x4*>(src + (int64_t)c * 16) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v[E];
                widen(In{}, d[u], v);
#pragma unroll
                for (int e = 0; e < E; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
            }
        }
    }
    am = block_max(am, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = am;
}

template <class In>
__global__ __launch_bounds__(kThreads) void tw_quant_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                            int M, int cpr, const float* __restrict__ partial,
                                                            int G, int8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ scale) {
    constexpr int E = In::E;
    __shared__ float red[kThreads / 64];
    float am = 0.0f;
    for (int i = threadIdx.x; i < G; i += kThreads) am = __builtin_fmaxf(am, partial[i]);
    am = block_max(am, red);
    const float s = am / 127.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
    // 0 = all codes zero, 1 = fast path with exact fallback, 2 = exact division everywhere
    const int mode = (s >= kSlowScale) ? 1 : (s == 0.0f ? 0 : 2);
    const float r = 1.0f / s;

    for (int i = blockIdx.x; i < M; i += gridDim.x) {
        const int row = M - 1 - i;
        const uint8_t* src = x + (int64_t)row * ldx_bytes;
        int8_t* dst = q + (int64_t)row * ldq;
        for (int c0 = 0; c0 < cpr; c0 += U * kThreads) {
            u32x4 d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kThreads + (int)threadIdx.x;
                d[u] = c < cpr ? *reinterpret_cast<const u32x4*>(src + (int64_t)c * 16) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kThreads + (int)threadIdx.x;
                if (c >= cpr) continue;
                float v[E];
                widen(In{}, d[u], v);
                uint32_t code[E];
                float dmax = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float t = __builtin_fmaf(v[e], r, kMagic);
                    const float n = t - kMagic;
                    const float dd = __builtin_fmaf(v[e], r, -n);
                    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(dd));
                    code[e] = f_bits(t);
                }
                if (__builtin_expect(mode != 1 || dmax >= kFastMargin, 0)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float t = __builtin_fmaf(v[e], r, kMagic);
                        const float n = t - kMagic;
                        const float dd = __builtin_fmaf(v[e], r, -n);
                        if (mode != 1 || __builtin_fabsf(dd) >= kFastMargin)
                            code[e] = mode == 0 ? 0u : exact_code<false, 127>(v[e], 1.0f, s);
                    }
                }
                if (E == 8) {
                    const u32x2 p = {pack4(code[0], code[1], code[2], code[3]),
                                     pack4(code[4 % E], code[5 % E], code[6 % E], code[7 % E])};
                    __builtin_nontemporal_store(p, reinterpret_cast<u32x2*>(dst + (int64_t)c * E));
                } else {
                    __builtin_nontemporal_store(pack4(code[0], code[1], code[2], code[3]),
                                                reinterpret_cast<uint32_t*>(dst + (int64_t)c * E));
                }
            }
        }
    }
}

template <class In>
hipError_t launch_tw(const void* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                     float* partial, hipStream_t stream) {
    constexpr int ESZ = 16 / In::E;
    const int cpr = (int)(K / In::E);                       // K % 16 == 0
    const int G = (int)(M < kTensorwisePartials ? M : kTensorwisePartials);
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    tw_amax_kernel<In><<<dim3(G), dim3(kThreads), 0, stream>>>(xb, ldx * ESZ, (int)M, cpr, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    tw_quant_kernel<In><<<dim3(G), dim3(kThreads), 0, stream>>>(xb, ldx * ESZ, (int)M, cpr, partial, G, q, ldq,
                                                               scale);
    return hipGetLastError();
}

// Partial maxima of the allocation-free entry point: kTensorwisePartials
// floats (8 KB), one copy per GPU, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it passes the device address looked up below.
static __device__ __align__(256) float scratch[kTensorwisePartials];

constexpr int kMaxDevices = 64;

}  // namespace

// Device address of `scratch` on the GPU that runs `stream`, looked up with
// hipGetSymbolAddress once per device (that device current) and cached.
hipError_t tensorwise_scratch(hipStream_t stream, float** out, size_t* floats) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    // the null stream runs on the calling thread's current device
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float*>(p);
    }
    *out = addr[dev];
    *floats = kTensorwisePartials;
    return hipSuccess;
}

hipError_t launch_quant_tensorwise(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                   int64_t ldq, float* scale, float* partial, hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_tw<InF32>(x, M, K, ldx, q, ldq, scale, partial, stream);
        case 1: return launch_tw<InBF16>(x, M, K, ldx, q, ldq, scale, partial, stream);
        default: return launch_tw<InF16>(x, M, K, ldx, q, ldq, scale, partial, stream);
    }
}

}  // namespace qd
