// ssd_api.hip -- the SSD prefill entry points declared in include/ssd.h:
// host-side validation of the argument struct (never of device data), the
// workspace layout, the kernel launches, and the static scratch of the entry
// point that allocates nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ssd.h"
#include "ssd_kernel.hpp"
#include "ssd_launch.h"
#include "ssu_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t s16, cb, cumlast, head, next, desc, w, cv, runs, wfirst, wlen, winfo, total;
};

Layout layout(int64_t nchunks, int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
              int64_t ngroups, int64_t chunk_size) {
    Layout l;
    l.s16 = 0;
    l.cb = l.s16 + round_up(static_cast<size_t>(nchunks * nheads * headdim * dstate) *
                            ssd::kEnterBytes);
    l.cumlast = l.cb + round_up(static_cast<size_t>(nchunks * ngroups * chunk_size * chunk_size) * 4);
    l.head = l.cumlast + round_up(static_cast<size_t>(nchunks * nheads) * 4);
    l.next = l.head + round_up(static_cast<size_t>(nchunks) * 4);
    l.desc = l.next + round_up(static_cast<size_t>(batch) * 4);
    l.w = l.desc + round_up(static_cast<size_t>(nchunks) * sizeof(ssd::ChunkDesc));
    l.cv = l.w + round_up(static_cast<size_t>(nchunks * nheads * chunk_size) * 4);
    l.runs = l.cv + round_up(static_cast<size_t>(nchunks * nheads * chunk_size) * 8);
    l.wfirst = l.runs + round_up(static_cast<size_t>(nchunks) * 4);
    l.wlen = l.wfirst + round_up(static_cast<size_t>(nchunks) * 4);
    l.winfo = l.wlen + round_up(static_cast<size_t>(nchunks) * 4);
    l.total = l.winfo + round_up(4);
    return l;
}

bool is_dtype(int32_t d) { return d == SSU_F32 || d == SSU_F16 || d == SSU_BF16; }
size_t dtype_size(int32_t d) { return d == SSU_F32 ? 4 : 2; }

struct Span {
    const char* name;
    const void* p;
    size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int check(const ssu_ssd_args& a) {
    using ssu::report;
    if (a.reserved != 0) return report(SSU_ERR_INVALID_ARGUMENT, "reserved must be 0");
    if (a.tokens < 0 || a.nheads < 1 || a.headdim < 1 || a.dstate < 1 || a.ngroups < 1)
        return report(SSU_ERR_INVALID_ARGUMENT,
                      "sizes must be positive (tokens %lld, heads %lld, headdim %lld, "
                      "dstate %lld, groups %lld)",
                      (long long)a.tokens, (long long)a.nheads, (long long)a.headdim,
                      (long long)a.dstate, (long long)a.ngroups);
    if (a.nheads % a.ngroups)
        return report(SSU_ERR_INVALID_ARGUMENT, "nheads (%lld) must be divisible by ngroups (%lld)",
                      (long long)a.nheads, (long long)a.ngroups);
    if (a.chunk_size < 1) return report(SSU_ERR_INVALID_ARGUMENT, "chunk_size must be positive");
    if (a.nchunks < 1)
        return report(SSU_ERR_INVALID_ARGUMENT, "cu_chunk_seqlens must have at least two entries");
    if (a.batch < 0) return report(SSU_ERR_INVALID_ARGUMENT, "batch must be >= 0");
    if (a.io_dtype != SSU_F16 && a.io_dtype != SSU_BF16)
        return report(SSU_ERR_INVALID_ARGUMENT, "x, B and C must share one of fp16/bf16");
    if (!is_dtype(a.dt_dtype))
        return report(SSU_ERR_INVALID_ARGUMENT, "dt must be fp32, fp16 or bf16");
    if (!is_dtype(a.state_dtype))
        return report(SSU_ERR_INVALID_ARGUMENT, "state_dtype must be fp16, bf16 or fp32");
    if (a.meta_dtype != SSU_I32 && a.meta_dtype != SSU_I64)
        return report(SSU_ERR_INVALID_ARGUMENT, "chunk metadata must be int32 or int64");
    if (!(a.dt_min <= a.dt_max))
        return report(SSU_ERR_INVALID_ARGUMENT, "dt_limit must satisfy min <= max");
    if (a.tokens > 0 && (!a.x || !a.dt || !a.B || !a.C || !a.out))
        return report(SSU_ERR_INVALID_ARGUMENT, "x, dt, B, C and out are required");
    if (!a.A) return report(SSU_ERR_INVALID_ARGUMENT, "A is required");
    if (!a.cu_chunk_seqlens || !a.seq_idx)
        return report(SSU_ERR_INVALID_ARGUMENT, "cu_chunk_seqlens and seq_idx are required");
    if (a.batch > 0 && !a.last_chunk_indices)
        return report(SSU_ERR_INVALID_ARGUMENT, "last_chunk_indices is required");
    const int64_t rows_out = a.return_intermediate_states ? a.nchunks : a.batch;
    if (rows_out > 0 && !a.states) return report(SSU_ERR_INVALID_ARGUMENT, "states is required");
    if (!ssd::supported_shape(a.headdim, a.dstate, a.chunk_size))
        return report(SSU_ERR_UNSUPPORTED,
                      "no kernel for headdim %lld, dstate %lld, chunk_size %lld (built: headdim "
                      "64, 128, 192 or 256, dstate 64, 128 or 256, chunk_size 128 or 256)",
                      (long long)a.headdim, (long long)a.dstate, (long long)a.chunk_size);
    if (a.nchunks * a.nheads * (a.headdim / 64) > INT32_MAX || a.nchunks * a.ngroups * 16 > INT32_MAX)
        return report(SSU_ERR_UNSUPPORTED, "too many chunks for one launch");
    // The kernels address a chunk's rows with 32-bit byte offsets.
    if (a.chunk_size * a.nheads * a.headdim * 2 >= (int64_t(1) << 30) ||
        a.chunk_size * a.ngroups * a.dstate * 2 >= (int64_t(1) << 30))
        return report(SSU_ERR_UNSUPPORTED, "a chunk's rows must span less than 1 GiB");
    for (const Span& s : {Span{"x", a.x, 0}, Span{"B", a.B, 0}, Span{"C", a.C, 0},
                          Span{"z", a.z, 0}, Span{"out", a.out, 0}})
        if (s.p && !aligned(s.p, 16))
            return report(SSU_ERR_UNSUPPORTED, "%s must be 16-byte aligned", s.name);
    const size_t ssz = dtype_size(a.state_dtype);
    if (a.initial_states && !aligned(a.initial_states, ssz))
        return report(SSU_ERR_UNSUPPORTED, "initial_states must be aligned to its element size");
    if (a.states && !aligned(a.states, 16))
        return report(SSU_ERR_UNSUPPORTED, "states must be 16-byte aligned");
    const Layout l = layout(a.nchunks, a.batch, a.nheads, a.headdim, a.dstate, a.ngroups,
                            a.chunk_size);
    if (!a.workspace || !aligned(a.workspace, kAlign) || a.workspace_bytes < l.total)
        return report(SSU_ERR_INVALID_ARGUMENT,
                      "workspace must be 256-byte aligned and hold %zu bytes (got %zu)", l.total,
                      a.workspace_bytes);

    const size_t T = static_cast<size_t>(a.tokens), H = a.nheads, P = a.headdim, N = a.dstate,
                 G = a.ngroups;
    const size_t io = 2, tile = H * P * N * ssz;
    const Span out{"out", a.out, T * H * P * io};
    const Span states{"states", a.states, static_cast<size_t>(rows_out) * tile};
    const Span ws{"workspace", a.workspace, l.total};
    const Span inputs[] = {
        {"x", a.x, T * H * P * io},
        {"dt", a.dt, T * H * dtype_size(a.dt_dtype)},
        {"A", a.A, H * 4},
        {"B", a.B, T * G * N * io},
        {"C", a.C, T * G * N * io},
        {"D", a.D, (a.D_per_dim ? H * P : H) * 4},
        {"z", a.z, a.z ? T * H * P * io : 0},
        {"dt_bias", a.dt_bias, a.dt_bias ? H * 4 : 0},
        {"initial_states", a.initial_states,
         a.initial_states ? static_cast<size_t>(a.batch) * tile : 0},
        {"cu_chunk_seqlens", a.cu_chunk_seqlens,
         static_cast<size_t>(a.nchunks + 1) * (a.meta_dtype == SSU_I64 ? 8 : 4)},
        {"seq_idx", a.seq_idx, static_cast<size_t>(a.nchunks) * (a.meta_dtype == SSU_I64 ? 8 : 4)},
        {"last_chunk_indices", a.last_chunk_indices,
         static_cast<size_t>(a.batch) * (a.meta_dtype == SSU_I64 ? 8 : 4)},
    };
    for (const Span& w : {out, states, ws}) {
        for (const Span& in : inputs)
            if (overlap(w, in))
                return report(SSU_ERR_INVALID_ARGUMENT, "%s overlaps %s", w.name, in.name);
    }
    if (overlap(out, states) || overlap(out, ws) || overlap(states, ws))
        return report(SSU_ERR_INVALID_ARGUMENT, "out, states and workspace must not overlap");
    return SSU_OK;
}

}  // namespace

extern "C" size_t ssu_ssd_workspace_bytes(int64_t nchunks, int64_t batch, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int64_t ngroups,
                                          int64_t chunk_size) {
    if (nchunks < 0 || batch < 0 || nheads < 0 || headdim < 0 || dstate < 0 || ngroups < 0 ||
        chunk_size < 0)
        return 0;
    return layout(nchunks, batch, nheads, headdim, dstate, ngroups, chunk_size).total;
}

namespace {

// The launches of one validated prefill, with a.workspace as its scratch.
int launch(const ssu_ssd_args& a, void* stream) {
    const Layout l = layout(a.nchunks, a.batch, a.nheads, a.headdim, a.dstate, a.ngroups,
                            a.chunk_size);
    char* ws = static_cast<char*>(a.workspace);
    ssd::SsdParams p{};
    p.x = a.x;
    p.dt = a.dt;
    p.A = a.A;
    p.B = a.B;
    p.C = a.C;
    p.D = a.D;
    p.z = a.z;
    p.dt_bias = a.dt_bias;
    p.cu_chunk = a.cu_chunk_seqlens;
    p.seq_idx = a.seq_idx;
    p.lci = a.last_chunk_indices;
    p.init = a.initial_states;
    p.out = a.out;
    p.states = a.states;
    p.s16 = ws + l.s16;
    p.cb = reinterpret_cast<float*>(ws + l.cb);
    p.cumlast = reinterpret_cast<float*>(ws + l.cumlast);
    p.list_head = reinterpret_cast<int*>(ws + l.head);
    p.list_next = reinterpret_cast<int*>(ws + l.next);
    p.desc = reinterpret_cast<ssd::ChunkDesc*>(ws + l.desc);
    p.w = reinterpret_cast<float*>(ws + l.w);
    p.cv = reinterpret_cast<float*>(ws + l.cv);
    p.run_first = reinterpret_cast<int*>(ws + l.runs);
    p.walk_first = reinterpret_cast<int*>(ws + l.wfirst);
    p.walk_len = reinterpret_cast<int*>(ws + l.wlen);
    p.walk_info = reinterpret_cast<int*>(ws + l.winfo);
    p.tokens = a.tokens;
    p.nchunks = a.nchunks;
    p.batch = a.batch;
    p.dt_min = static_cast<float>(a.dt_min);
    p.dt_max = static_cast<float>(a.dt_max);
    p.nheads = static_cast<int32_t>(a.nheads);
    p.ngroups = static_cast<int32_t>(a.ngroups);
    p.heads_per_group = static_cast<int32_t>(a.nheads / a.ngroups);
    p.headdim = static_cast<int32_t>(a.headdim);
    p.dstate = static_cast<int32_t>(a.dstate);
    p.dt_dtype = a.dt_dtype;
    p.meta_i64 = a.meta_dtype == SSU_I64;
    p.D_per_dim = a.D_per_dim != 0;
    p.dt_softplus = a.dt_softplus != 0;
    p.return_all = a.return_intermediate_states != 0;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int P = static_cast<int>(a.headdim), N = static_cast<int>(a.dstate),
              Q = static_cast<int>(a.chunk_size);
    const hipError_t err = a.io_dtype == SSU_BF16
                               ? ssd::launch_ssd_bf16(p, a.state_dtype, P, N, Q, s)
                               : ssd::launch_ssd_f16(p, a.state_dtype, P, N, Q, s);
    if (err != hipSuccess)
        return ssu::report(SSU_ERR_LAUNCH, "SSD prefill launch failed: %s", hipGetErrorString(err));
    return ssu::report_ok();
}

}  // namespace

// Scratch of ssu_ssd_prefill_noalloc: one array per GPU, placed by the loader
// with the library's device code and held until the process ends. In host code
// `scratch` is only a handle for the symbol, never a device address: its device
// address is looked up once per device (with that device current) and kept in
// scratch_ptr, which is what kernels and copies receive.
constexpr size_t kStaticScratch = SSU_SSD_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratch % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) unsigned char scratch[kStaticScratch];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up on its first use there.
int current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ssu::report(SSU_ERR_LAUNCH, "no usable current HIP device (%d)", dev);
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return ssu::report(SSU_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s",
                               dev, hipGetErrorString(e));
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return SSU_OK;
}

}  // namespace

extern "C" int ssu_ssd_prefill(const ssu_ssd_args* args, void* stream) {
    if (!args) return ssu::report(SSU_ERR_INVALID_ARGUMENT, "args is NULL");
    if (args->struct_size != sizeof(ssu_ssd_args))
        return ssu::report(SSU_ERR_INVALID_ARGUMENT, "struct_size %u, expected %zu",
                           args->struct_size, sizeof(ssu_ssd_args));
    const ssu_ssd_args& a = *args;
    if (const int rc = check(a)) return rc;
    return launch(a, stream);
}

extern "C" int ssu_ssd_prefill_noalloc(const ssu_ssd_args* args, void* stream) {
    if (!args) return ssu::report(SSU_ERR_INVALID_ARGUMENT, "args is NULL");
    if (args->struct_size != sizeof(ssu_ssd_args))
        return ssu::report(SSU_ERR_INVALID_ARGUMENT, "struct_size %u, expected %zu",
                           args->struct_size, sizeof(ssu_ssd_args));
    if (args->workspace || args->workspace_bytes)
        return ssu::report(SSU_ERR_INVALID_ARGUMENT,
                           "workspace must be NULL and workspace_bytes 0: this entry point uses "
                           "the library's static scratch");
    // Sizes first (host arithmetic only), then the device's scratch.
    if (args->nchunks >= 0 && args->batch >= 0 && args->nheads >= 0 && args->headdim >= 0 &&
        args->dstate >= 0 && args->ngroups >= 0 && args->chunk_size >= 0) {
        const size_t need = layout(args->nchunks, args->batch, args->nheads, args->headdim,
                                   args->dstate, args->ngroups, args->chunk_size).total;
        if (need > kStaticScratch)
            return ssu::report(SSU_ERR_UNSUPPORTED,
                               "this prefill needs %zu bytes of scratch; the static scratch holds "
                               "%zu (SSU_SSD_STATIC_SCRATCH_BYTES): pass a workspace to "
                               "ssu_ssd_prefill instead",
                               need, kStaticScratch);
    }
    ssu_ssd_args a = *args;
    if (a.nheads >= 1 && a.headdim >= 1 && a.dstate >= 1 && a.ngroups >= 1 && a.nchunks >= 1) {
        if (const int rc = current_scratch(&a.workspace)) return rc;
        a.workspace_bytes = kStaticScratch;
    }
    if (const int rc = check(a)) return rc;
    return launch(a, stream);
}
