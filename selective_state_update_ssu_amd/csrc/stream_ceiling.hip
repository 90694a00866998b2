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

}  // extern "C"
