// stream_ceiling.hip -- plain streaming kernels that measure what HBM sustains
// for a given read/write mix on this GPU. Built into a separate library
// (libssu_stream.so) used by the benchmark only: a copy of known size for
// calibrating traffic counters, and read-only / write-only / copy ceilings to
// set the SSU kernel's achieved bandwidth against.
//
// Each thread moves UNROLL 16-byte vectors spaced one workgroup apart, so every
// wave instruction touches one contiguous 1 KiB run, as the SSU kernel does.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunk = size_t(kThreads) * kUnroll * sizeof(u32x4);  // bytes per workgroup

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src, size_t n) {
    const size_t base = size_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const size_t j = base + size_t(i) * kThreads;
        v[i] = j < n ? __builtin_nontemporal_load(src + j) : u32x4(0u);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const size_t j = base + size_t(i) * kThreads;
        if (j < n) __builtin_nontemporal_store(v[i], dst + j);
    }
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        unsigned* __restrict__ sink) {
    const size_t base = size_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
    u32x4 acc = u32x4(0u);
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const size_t j = base + size_t(i) * kThreads;
        if (j < n) acc ^= __builtin_nontemporal_load(src + j);
    }
    // The xor of the data is never this value for buffers the benchmark fills;
    // the store keeps the loads alive without adding traffic.
    if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[blockIdx.x & 1023] = acc.z;
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* __restrict__ dst, size_t n,
                                                         unsigned value) {
    const size_t base = size_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
        const size_t j = base + size_t(i) * kThreads;
        if (j < n) __builtin_nontemporal_store(u32x4(value), dst + j);
    }
}

// The state traffic of a packed multi-token call without its arithmetic: for
// every (sequence, head, block of the head's tile) the block is read once from
// the sequence's read slot and written to each valid destination slot of the
// sequence's table row, in the same order of workgroups as the SSU kernel. Four
// heads per workgroup, two 16-byte vectors per lane, non-temporal: the fastest
// of the shapes tried for this pattern.
constexpr int kFanHeads = 4;
constexpr int kFanLoads = 2;
constexpr size_t kFanBlock = size_t(kThreads) * kFanLoads * sizeof(u32x4);  // bytes per head

struct FanParams {
    char* state;
    size_t slot_bytes, head_bytes;
    const int* table;    // [nseq, steps]
    const int* accepted; // [nseq], entries in [1, steps]
    const int* starts;   // [nseq + 1]
    int nslots, steps, head_blocks, tile_blocks;
};

__global__ __launch_bounds__(kThreads* kFanHeads) void fanout_kernel(const FanParams p) {
    const int tid = threadIdx.x;
    const int lh = __builtin_amdgcn_readfirstlane(tid / kThreads);
    const int ht = tid % kThreads;
    int64_t wg = blockIdx.x;
    const int tb = static_cast<int>(wg % p.tile_blocks);
    wg /= p.tile_blocks;
    const int64_t h = (wg % p.head_blocks) * kFanHeads + lh;
    const int64_t seq = wg / p.head_blocks;
    const int len = p.starts[seq + 1] - p.starts[seq];
    const int k = p.accepted[seq];
    if (k < 1 || k > p.steps) return;
    const int r = __builtin_amdgcn_readfirstlane(p.table[seq * p.steps + k - 1]);
    if (r < 0 || r >= p.nslots) return;
    const size_t base = h * p.head_bytes + tb * kFanBlock;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.state + r * p.slot_bytes + base);
    u32x4 v[kFanLoads];
#pragma unroll
    for (int i = 0; i < kFanLoads; ++i) v[i] = __builtin_nontemporal_load(src + ht + i * kThreads);
    for (int t = 0; t < len && t < p.steps; ++t) {
        const int w = __builtin_amdgcn_readfirstlane(p.table[seq * p.steps + t]);
        if (w < 0 || w >= p.nslots) continue;
        u32x4* dst = reinterpret_cast<u32x4*>(p.state + w * p.slot_bytes + base);
#pragma unroll
        for (int i = 0; i < kFanLoads; ++i) __builtin_nontemporal_store(v[i], dst + ht + i * kThreads);
    }
}

dim3 grid_for(size_t bytes) { return dim3(static_cast<unsigned>((bytes + kChunk - 1) / kChunk)); }

int finish() { return hipGetLastError() == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {

// All sizes in bytes, multiples of 16; pointers 16-byte aligned device memory.
// `sink` must hold 1024 unsigned. Each returns 0 on a successful launch.
int ssu_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(copy_kernel, grid_for(bytes), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                       static_cast<const u32x4*>(src), bytes / 16);
    return finish();
}

int ssu_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(read_kernel, grid_for(bytes), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, static_cast<unsigned*>(sink));
    return finish();
}

int ssu_stream_write(void* dst, size_t bytes, void* stream) {
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(write_kernel, grid_for(bytes), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst), bytes / 16,
                       0x3F800000u);
    return finish();
}

// Packed-call state traffic (fanout_kernel) over a state cache of `nslots` slots
// of `nheads` heads of `head_bytes` bytes each. Int32 device arrays: table
// [nseq, steps], accepted [nseq], starts [nseq + 1]. Returns 2 when nheads is
// not a multiple of 4 or head_bytes not a multiple of 8 KiB (the kernel's
// blocking), 0 on a successful launch.
int ssu_stream_fanout(void* state, int64_t nslots, int64_t nheads, size_t head_bytes,
                      const void* table, int64_t steps, const void* accepted,
                      const void* starts, int64_t nseq, void* stream) {
    if (nheads % kFanHeads || head_bytes % kFanBlock || nslots <= 0 || steps <= 0) return 2;
    if (nseq == 0) return 0;
    FanParams p;
    p.state = static_cast<char*>(state);
    p.slot_bytes = head_bytes * nheads;
    p.head_bytes = head_bytes;
    p.table = static_cast<const int*>(table);
    p.accepted = static_cast<const int*>(accepted);
    p.starts = static_cast<const int*>(starts);
    p.nslots = static_cast<int>(nslots);
    p.steps = static_cast<int>(steps);
    p.head_blocks = static_cast<int>(nheads / kFanHeads);
    p.tile_blocks = static_cast<int>(head_bytes / kFanBlock);
    const dim3 grid(static_cast<unsigned>(nseq * p.head_blocks * p.tile_blocks));
    hipLaunchKernelGGL(fanout_kernel, grid, dim3(kThreads * kFanHeads), 0,
                       static_cast<hipStream_t>(stream), p);
    return finish();
}

}  // extern "C"
