// Kernel instances for float state storage (every io dtype and dstate).
#include "ssu_kernel.hpp"

namespace ssu {

hipError_t launch_state_f32(const KernelParams& p, int io_dtype, int dstate, dim3 grid,
                           dim3 block, hipStream_t stream) {
    return launch_state<float>(p, io_dtype, dstate, grid, block, stream);
}

}  // namespace ssu
