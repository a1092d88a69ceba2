// Host-only stand-ins for the kernel launchers of qd_launch.h, for building
// the C ABI's argument checks (capi.cpp) with AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU.  Each launcher returns success
// without touching its pointers (the tests pass placeholder addresses), so
// every path through capi.cpp can run with no GPU.
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "qd_launch.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "placeholder HIP error"; }

namespace qd {

hipError_t launch_rotquant(const void*, int, bool, int, int64_t, int64_t, int64_t, int8_t*, int64_t, float*,
                           hipStream_t, int) { return hipSuccess; }
hipError_t launch_rotquant_sliced(const void*, int, int64_t, int64_t, int64_t, int8_t*, float*, hipStream_t, int) {
    return hipSuccess;
}
hipError_t launch_rotquant_fp6(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, hipStream_t,
                               bool) { return hipSuccess; }
hipError_t launch_input_act(const void*, int, int64_t, int, void*, hipStream_t) { return hipSuccess; }
hipError_t launch_quant_tensorwise(const void*, int, int64_t, int64_t, int64_t, int8_t*, int64_t, float*, float*,
                                   hipStream_t) { return hipSuccess; }
hipError_t tensorwise_scratch(hipStream_t, float** partial, size_t* floats) {
    static float placeholder[kTensorwisePartials];
    *partial = placeholder;
    *floats = kTensorwisePartials;
    return hipSuccess;
}
hipError_t launch_attention_i8(const int8_t*, const float*, const int8_t*, const float*, const int8_t*, const float*,
                               void*, int64_t, int64_t, int64_t, int64_t, float, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_bf16(const int8_t*, int64_t, const float*, const int8_t*, int64_t, const float*, const void*,
                            void*, int64_t, int64_t, int64_t, int64_t, hipStream_t, int, int, bool, bool) {
    return hipSuccess;
}
hipError_t launch_gemm_i32(const int8_t*, int64_t, const int8_t*, int64_t, int32_t*, int64_t, int64_t, int64_t,
                           int64_t, hipStream_t, bool, bool) { return hipSuccess; }
hipError_t launch_slice_weights(const int8_t*, int64_t, int64_t, int64_t, int8_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_w4_bf16(const int8_t*, int64_t, const float*, const uint8_t*, int64_t, const float*,
                               const void*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t, int, int) {
    return hipSuccess;
}
hipError_t launch_gemm_w4_i32(const int8_t*, int64_t, const uint8_t*, int64_t, int32_t*, int64_t, int64_t, int64_t,
                              int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_pack_int4(const int8_t*, int64_t, uint8_t*, int64_t, int64_t, int64_t, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_pack_fp6(const int8_t*, int64_t, uint8_t*, int64_t, int64_t, int64_t, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_gemm_f6_bf16(const uint8_t*, int64_t, const float*, const uint8_t*, int64_t, const float*,
                               const void*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t, bool, bool) {
    return hipSuccess;
}
hipError_t launch_gemm_f6_i32(const uint8_t*, int64_t, const uint8_t*, int64_t, int32_t*, int64_t, int64_t, int64_t,
                              int64_t, hipStream_t, bool, bool) { return hipSuccess; }
hipError_t launch_slice_fp6(const uint8_t*, int64_t, int64_t, int64_t, uint8_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_dequant(const int8_t*, int64_t, const float*, bool, bool, void*, int64_t, int64_t, int64_t,
                          hipStream_t) { return hipSuccess; }

}  // namespace qd
