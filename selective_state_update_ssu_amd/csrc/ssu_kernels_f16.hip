// Kernel instances for _Float16 state storage (every io dtype and dstate).
#include "ssu_kernel.hpp"

namespace ssu {

hipError_t launch_state_f16(const KernelParams& p, int io_dtype, int dstate, dim3 grid,
                           dim3 block, hipStream_t stream) {
    return launch_state<_Float16>(p, io_dtype, dstate, grid, block, stream);
}

}  // namespace ssu
