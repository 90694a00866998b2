// Kernel instances for _Float16 state storage (every io dtype and dstate).
#include "ssu_kernel.hpp"

namespace ssu {

hipError_t launch_state_f16(KernelParams p, int io_dtype, int dstate, int64_t nseq,
                           hipStream_t stream, LaunchShape* shape) {
    return launch_state<_Float16>(p, io_dtype, dstate, nseq, stream, shape);
}

}  // namespace ssu
