// Kernel instances for __bf16 state storage (every io dtype and dstate).
#include "ssu_kernel.hpp"

namespace ssu {

hipError_t launch_state_bf16(const KernelParams& p, int io_dtype, int dstate, dim3 grid,
                           dim3 block, hipStream_t stream) {
    return launch_state<__bf16>(p, io_dtype, dstate, grid, block, stream);
}

}  // namespace ssu
