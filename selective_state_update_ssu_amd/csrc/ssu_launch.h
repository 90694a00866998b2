// ssu_launch.h -- internal interface between the C-ABI front end (ssu_api.hip)
// and the per-state-dtype kernel translation units. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssu {

// Rows of one head covered by one 256-thread head group of a workgroup.
constexpr int kRowsPerBlock = 64;
// Threads per head group (four wave64s).
constexpr int kHeadThreads = 256;
// Largest number of heads one workgroup may cover.
constexpr int kMaxHeadsPerBlock = 4;

// Heads per workgroup a dstate allows: dstate 256 keeps 64 state values per lane,
// so its workgroups stop at 512 threads to leave the compiler 256 VGPRs.
__host__ __device__ constexpr int max_heads_per_block(int dstate) {
    return dstate >= 256 ? 2 : kMaxHeadsPerBlock;
}

// Everything a launch needs, by value. Sizes are validated on the host.
struct KernelParams {
    void* state;
    const void* x;
    const void* B;
    const void* C;
    const void* z;      // may be null
    void* out;
    const float* dt;
    const float* A;
    const float* D;        // may be null
    const float* dt_bias;  // may be null

    // Slot resolution.
    const void* src;    // one-token: [batch] vector; packed: table; may be null
    const void* dst;    // may be null
    const void* cu;     // packed only
    const void* na;     // packed only, may be null
    int64_t src_seq_stride, src_step_stride;
    int64_t dst_seq_stride, dst_step_stride;
    int64_t steps;
    int64_t nslots;
    int64_t pad_slot_id;
    int64_t rows;

    int32_t nheads, headdim, ngroups, heads_per_group;
    int32_t heads_per_block;  // heads per workgroup (same group)
    int32_t head_blocks;      // nheads / heads_per_block
    int32_t row_blocks;       // ceil(headdim / kRowsPerBlock)

    int32_t src_i64, dst_i64, meta_i64;
    int32_t packed;
    int32_t dt_per_dim;
    int32_t dt_softplus;
    int32_t disable_state_update;
};

// One launcher per state dtype; each dispatches on (io dtype, dstate).
// Returns hipErrorInvalidValue for an (io, dstate) pair it was not built for.
hipError_t launch_state_f32(const KernelParams& p, int io_dtype, int dstate,
                            dim3 grid, dim3 block, hipStream_t stream);
hipError_t launch_state_f16(const KernelParams& p, int io_dtype, int dstate,
                            dim3 grid, dim3 block, hipStream_t stream);
hipError_t launch_state_bf16(const KernelParams& p, int io_dtype, int dstate,
                             dim3 grid, dim3 block, hipStream_t stream);

}  // namespace ssu
