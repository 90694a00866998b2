// ring_trackers.hip -- ReplaySSM ring-tracker update/reset and delayed commit
// (semantics in include/ssu.h). One thread per position; every load and store
// of a counter is guarded by the validity of the position's slot. Integer only.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ssu.h"
#include "ssu_launch.h"

namespace {

constexpr int kThreads = 256;

struct RingParams {
    void* ring_start;
    void* prev_num_accepted;
    void* prev_query_len;
    const void* slots;
    const void* num_accepted;
    const void* query_start_loc;
    int64_t num_states, slot_stride, n;
    int64_t logical_window, ring_buffer_len, pad_slot_id;
    int32_t t64, s64, m64;
};

__device__ __forceinline__ int64_t ld(const void* p, int is64, int64_t i) {
    return is64 ? static_cast<const int64_t*>(p)[i]
                : static_cast<int64_t>(static_cast<const int32_t*>(p)[i]);
}

__device__ __forceinline__ void st(void* p, int is64, int64_t i, int64_t v) {
    if (is64)
        static_cast<int64_t*>(p)[i] = v;
    else
        static_cast<int32_t*>(p)[i] = static_cast<int32_t>(v);
}

enum Mode { kReset = 0, kAdvance = 1, kCommit = 2 };

template <int MODE>
__global__ __launch_bounds__(kThreads) void ring_kernel(const RingParams p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= p.n) return;
    const int64_t s = ld(p.slots, p.s64, i * p.slot_stride);
    if (s == p.pad_slot_id || s < 0 || s >= p.num_states) return;
    if constexpr (MODE == kReset) {
        st(p.ring_start, p.t64, s, 0);
        st(p.prev_num_accepted, p.t64, s, 0);
        st(p.prev_query_len, p.t64, s, 0);
    } else if constexpr (MODE == kAdvance) {
        const int64_t counted = ld(p.prev_num_accepted, p.t64, s);
        if (counted + 1 > p.logical_window) {
            const int64_t start = ld(p.ring_start, p.t64, s);
            st(p.ring_start, p.t64, s, (start + counted) % p.ring_buffer_len);
            st(p.prev_num_accepted, p.t64, s, 1);
        } else {
            st(p.prev_num_accepted, p.t64, s, counted + 1);
        }
    } else {
        const int64_t counted = ld(p.prev_num_accepted, p.t64, s);
        const int64_t window = ld(p.prev_query_len, p.t64, s);
        const int64_t accepted = ld(p.num_accepted, p.m64, i);
        const int64_t qlen = ld(p.query_start_loc, p.m64, i + 1) - ld(p.query_start_loc, p.m64, i);
        if (window == 0) {
            st(p.prev_num_accepted, p.t64, s, 0);
        } else if (counted + window > p.logical_window) {
            const int64_t start = ld(p.ring_start, p.t64, s);
            st(p.ring_start, p.t64, s, (start + counted) % p.ring_buffer_len);
            st(p.prev_num_accepted, p.t64, s, accepted);
        } else {
            st(p.prev_num_accepted, p.t64, s, counted + accepted);
        }
        st(p.prev_query_len, p.t64, s, qlen);
    }
}

bool is_index(int32_t d) { return d == SSU_I32 || d == SSU_I64; }

int check(const ssu_ring_args* a, bool commit, bool reset) {
    using ssu::report;
    if (!a) return report(SSU_ERR_INVALID_ARGUMENT, "args must not be NULL");
    if (a->struct_size != sizeof(ssu_ring_args))
        return report(SSU_ERR_INVALID_ARGUMENT,
                      "struct_size %u != sizeof(ssu_ring_args) %zu (header mismatch)",
                      a->struct_size, sizeof(ssu_ring_args));
    if (a->n < 0 || a->num_states < 0)
        return report(SSU_ERR_INVALID_ARGUMENT, "n and num_states must be >= 0");
    if (a->slot_stride < 0) return report(SSU_ERR_INVALID_ARGUMENT, "slot_stride must be >= 0");
    if (!is_index(a->tracker_dtype))
        return report(SSU_ERR_INVALID_ARGUMENT, "tracker_dtype %d is not an ssu_index_dtype",
                      a->tracker_dtype);
    if (!is_index(a->slot_dtype))
        return report(SSU_ERR_INVALID_ARGUMENT, "slot_dtype %d is not an ssu_index_dtype",
                      a->slot_dtype);
    if (commit && !is_index(a->meta_dtype))
        return report(SSU_ERR_INVALID_ARGUMENT, "meta_dtype %d is not an ssu_index_dtype",
                      a->meta_dtype);
    if (!reset && a->ring_buffer_len < 1)
        return report(SSU_ERR_INVALID_ARGUMENT, "ring_buffer_len must be >= 1, got %lld",
                      (long long)a->ring_buffer_len);
    if (!reset && a->logical_window < 0)
        return report(SSU_ERR_INVALID_ARGUMENT, "logical_window must be >= 0");
    if (a->n == 0) return SSU_OK;
    if (!a->slots) return report(SSU_ERR_INVALID_ARGUMENT, "slots must not be NULL");
    if (!a->ring_start || !a->prev_num_accepted || !a->prev_query_len)
        return report(SSU_ERR_INVALID_ARGUMENT, "tracker pointers must not be NULL");
    if (commit && (!a->num_accepted || !a->query_start_loc))
        return report(SSU_ERR_INVALID_ARGUMENT,
                      "num_accepted and query_start_loc must not be NULL");
    const uintptr_t tal = a->tracker_dtype == SSU_I64 ? 8 : 4;
    for (const void* q : {static_cast<const void*>(a->ring_start),
                          static_cast<const void*>(a->prev_num_accepted),
                          static_cast<const void*>(a->prev_query_len)})
        if (reinterpret_cast<uintptr_t>(q) % tal)
            return report(SSU_ERR_INVALID_ARGUMENT, "tracker arrays must be aligned to their dtype");
    return SSU_OK;
}

template <int MODE>
int launch(const ssu_ring_args* a, void* stream, const char* entry) {
    RingParams p{a->ring_start,     a->prev_num_accepted, a->prev_query_len, a->slots,
                 a->num_accepted,   a->query_start_loc,   a->num_states,     a->slot_stride,
                 a->n,              a->logical_window,    a->ring_buffer_len, a->pad_slot_id,
                 a->tracker_dtype == SSU_I64, a->slot_dtype == SSU_I64, a->meta_dtype == SSU_I64};
    const uint64_t blocks = (static_cast<uint64_t>(a->n) + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffull)
        return ssu::report(SSU_ERR_UNSUPPORTED, "%s: n is too large for one launch", entry);
    hipLaunchKernelGGL(ring_kernel<MODE>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return ssu::report(SSU_ERR_LAUNCH, "%s: launch failed: %s", entry, hipGetErrorString(e));
    return ssu::report_ok();
}

}  // namespace

extern "C" {

int ssu_ring_update(const ssu_ring_args* a, void* stream) {
    const bool reset = a && a->reset;
    if (int rc = check(a, false, reset)) return rc;
    if (a->n == 0) return ssu::report_ok();
    return reset ? launch<kReset>(a, stream, "ssu_ring_update")
                 : launch<kAdvance>(a, stream, "ssu_ring_update");
}

int ssu_ring_commit(const ssu_ring_args* a, void* stream) {
    if (int rc = check(a, true, false)) return rc;
    if (a->n == 0) return ssu::report_ok();
    return launch<kCommit>(a, stream, "ssu_ring_commit");
}

}  // extern "C"
