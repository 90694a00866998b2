// SSD prefill kernels with bf16 x, B, C, z and out.
#include "ssd_kernel.hpp"
#include "ssd_launch.h"

hipError_t ssd::launch_ssd_bf16(const SsdParams& p, int state_dtype, int P, int N, int Q,
                                hipStream_t stream) {
    return launch_io<__bf16>(p, state_dtype, P, N, Q, stream);
}
