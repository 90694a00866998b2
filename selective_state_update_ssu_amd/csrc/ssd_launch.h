// ssd_launch.h -- internal interface between the SSD prefill entry point
// (ssd_api.hip) and its kernel translation units, one per io type. Not installed.
#pragma once

#include <hip/hip_runtime.h>

namespace ssd {

struct SsdParams;

// Headdim, dstate and chunk sizes with compiled kernels: headdim a multiple of
// 64 up to 256 (the kernels work on 64-column blocks), dstate 64, 128 or 256,
// chunks of 128 or 256 tokens.
inline bool supported_shape(int64_t P, int64_t N, int64_t Q) {
    return P >= 64 && P <= 256 && P % 64 == 0 && (N == 64 || N == 128 || N == 256) &&
           (Q == 128 || Q == 256);
}

// All launches of one prefill; hipErrorInvalidValue for an instance not built.
hipError_t launch_ssd_bf16(const SsdParams& p, int state_dtype, int P, int N, int Q,
                           hipStream_t stream);
hipError_t launch_ssd_f16(const SsdParams& p, int state_dtype, int P, int N, int Q,
                          hipStream_t stream);

}  // namespace ssd
