// ssu_launch.h -- internal interface between the C-ABI front end (ssu_api.hip)
// and the per-state-dtype kernel translation units. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssu {

// Depths of 16-byte state loads a lane may keep in flight; each is compiled. A
// lane gets fewer when a head's dstate rows are too short to give it that many.
constexpr int kLoadDepths[] = {2, 4};
// Largest number of heads one workgroup may cover.
constexpr int kMaxHeadsPerBlock = 4;

// Heads per workgroup an instance allows. Large states per lane (dstate 256) and
// the packed kernel (state plus a chunk of staged tokens) stop at two heads (512
// threads with four-wave head groups), to leave the compiler 256 VGPRs instead of
// spilling.
__host__ __device__ constexpr int max_heads_per_block(int dstate, bool packed) {
    return (dstate >= 256 || packed) ? 2 : kMaxHeadsPerBlock;
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
    const int64_t* rand_seed;  // may be null: round stored 16-bit states to nearest

    // Slot resolution.
    const void* src;    // one-token: [batch] vector; packed: table; may be null
    const void* dst;    // may be null
    const void* cu;     // packed only; null: regular sequences of seq_len rows
    const void* na;     // packed only, may be null
    int64_t src_seq_stride, src_step_stride;
    int64_t dst_seq_stride, dst_step_stride;
    int64_t steps;
    int64_t seq_len;
    int64_t nslots;
    int64_t pad_slot_id;
    int64_t rows;

    int32_t nheads, headdim, ngroups, heads_per_group;
    int32_t heads_per_block;  // heads per workgroup (same group)
    int32_t loads_per_lane;   // one of kLoadDepths
    int32_t xcd_order;        // 0: hardware order; 1: each XCD walks a contiguous range
                              // of tiles; 2: each XCD takes an equal contiguous share of
                              // every sequence's tiles
    int32_t head_blocks;      // nheads / heads_per_block
    int32_t row_blocks;       // ceil(headdim / rows per block), set by the launcher

    int32_t src_i64, dst_i64, meta_i64;
    int32_t packed;
    int32_t dt_per_dim;
    int32_t dt_softplus;
    int32_t disable_state_update;
    int32_t philox_rounds;
};

// Compute dies (XCDs) the hardware deals consecutive workgroups to, round robin.
constexpr int kXcds = 8;

// Launch shape chosen by a launcher (reported for logging).
struct LaunchShape {
    unsigned grid = 0, block = 0, lds_bytes = 0, rows_per_block = 0;
};

// One launcher per state dtype; each dispatches on (io dtype, dstate), derives
// the row block and grid of that kernel instance, and launches `nseq` sequences'
// worth of workgroups. Returns hipErrorInvalidValue for an (io, dstate) pair it
// was not built for and hipErrorInvalidConfiguration for a grid too large.
hipError_t launch_state_f32(KernelParams p, int io_dtype, int dstate, int64_t nseq,
                            hipStream_t stream, LaunchShape* shape);
hipError_t launch_state_f16(KernelParams p, int io_dtype, int dstate, int64_t nseq,
                            hipStream_t stream, LaunchShape* shape);
hipError_t launch_state_bf16(KernelParams p, int io_dtype, int dstate, int64_t nseq,
                             hipStream_t stream, LaunchShape* shape);

// Error reporting shared by every entry point of the library: set the calling
// thread's message and return `code` (report) or clear it and return 0 (ok).
int report(int code, const char* fmt, ...);
int report_ok();

}  // namespace ssu
