// ssd_kernel.hpp -- SSD chunked prefill for gfx950 (CDNA4, wave64, MFMA).
//
// The prefill of a Mamba-2 layer over packed variable-length requests, cut into
// chunks of at most Q tokens (semantics in include/ssd.h), as three launches:
//
//   front     three independent parts in one launch:
//     list    the requests whose last chunk is c, per chunk; the runs of chunks
//             that continue one another, longest first           (one workgroup)
//     prep    the chunk's descriptor; per (chunk, head) the clamped steps v_s,
//             the running sums cum_s and the weights exp(cum_last - cum_s) v_s
//     bmm     CB[t, s] = C_t . B_s                                 per (chunk, group, tile)
//   walk      S_c = exp(cum_last) S_{c-1} + sum_s w_s x_s B_s^T   per (run, head), in order
//   scan      y_t = sum_{s<=t} CB[t, s] exp(cum_t - cum_s) v_s x_s
//                   + exp(cum_t) C_t . S_{c-1} + D x_t, gated      per (chunk, head)
//
// with v the clamped step and cum the running sum of A v inside the chunk, in
// fp64. The walk's weights take exp of fp64 differences, exact to fp32 however
// far into the chunk; the scan's decays exp2 the difference of two fp32-rounded
// running sums (an absolute error of about one ulp of |cum| log2(e) in the
// exponent, far below the 16-bit rounding of the decayed entry for the
// magnitudes a chunk reaches). The three contractions run on the matrix cores with 16-bit
// operands and fp32 accumulation. Every operand that is not an input (the
// walk's w_s x_s, the scan's decayed C B^T entries and entering states) goes in
// as a high and a low 16-bit part, which makes each product accurate to about
// 2^-16 (bf16) or 2^-22 (fp16) instead of 2^-9 / 2^-12; x, B and C go in
// exactly. The walk keeps the state in its fp32 accumulators from chunk to
// chunk and hands each chunk's entering state to the scan as the two parts.
//
// Tiles are read through raw buffer descriptors whose range ends where the
// chunk's rows end: the hardware returns zeros past the range, so rows past a
// chunk's end need neither a branch nor a clamp, and every load of a tile is
// issued before the first of them is waited for.
//
// MFMA operand layouts (gfx950, checked on the hardware):
//   16x16x32: lane l holds A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16],
//             j < 8; the result D[4 (l / 16) + i][l % 16], i < 4.
//   32x32x16: lane l holds A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32];
//             the result D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i < 16.
// Both operands want eight consecutive values of the contracted index per lane.
// Where that index is the token, the token-major inputs are transposed on their
// way into LDS.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ssu_kernel.hpp"

namespace ssd {

using ssu::lds_barrier;
using ssu::load_index;

constexpr int kThreads = 256;  // four wave64s per workgroup
constexpr int kWaves = kThreads / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// dtype codes of include/ssu.h.
enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Per chunk, written by prep (in the front launch) for the later launches.
struct ChunkDesc {
    int64_t lo;     // first token
    int32_t len;    // tokens; 0 for an empty chunk or a range that is not valid
    int32_t enter;  // entering state: kEnterCarry (the previous chunk's), kEnterZero,
                    // or the row of the initial states
};
constexpr int32_t kEnterCarry = -2, kEnterZero = -1;

struct SsdParams {
    const void* x;        // [tokens, H, P] io
    const void* dt;       // [tokens, H] dt_dtype
    const float* A;       // [H]
    const void* B;        // [tokens, G, N] io
    const void* C;        // [tokens, G, N] io
    const float* D;       // [H] or [H, P], may be null
    const void* z;        // [tokens, H, P] io, may be null
    const float* dt_bias; // [H], may be null
    const void* cu_chunk; // [nchunks + 1]
    const void* seq_idx;  // [nchunks]
    const void* lci;      // [batch]
    const void* init;     // [batch, H, P, N] state type, may be null
    void* out;            // [tokens, H, P] io
    void* states;         // [nchunks or batch, H, P, N] state type
    void* s16;            // workspace [nchunks, H] tiles of kEnterBytes * P * N bytes: each
                          // chunk's entering state as [P, N] io-type high parts, then
                          // [P, N] low bytes
    float* cb;            // workspace [nchunks, G, Q, Q]
    float* cumlast;       // workspace [nchunks, H]: each chunk's decay exponent
    ChunkDesc* desc;      // workspace [nchunks]
    float* w;             // workspace [nchunks, H, Q]: chunk-state weights exp(cum_last - cum_s) v_s
    float* cv;            // workspace [nchunks, H, 2, Q]: cum_s log2(e) - log2(v_s), then
                          // cum_s log2(e), for the scan
    int* list_head;       // workspace [nchunks]: first request whose last chunk is c
    int* list_next;       // workspace [batch]
    int* run_first;       // workspace [nchunks]: first chunk of each run, in chunk order
    int* walk_first;      // workspace [nchunks]: runs by length, longest first: first chunk
    int* walk_len;        // workspace [nchunks]: and number of chunks
    int* walk_info;       // workspace [1]: number of runs
    int64_t tokens, nchunks, batch;
    float dt_min, dt_max;
    int32_t nheads, ngroups, heads_per_group;
    int32_t headdim, dstate;  // full sizes; the walk and the scan work on blocks of them
    int32_t dt_dtype;
    int32_t meta_i64;
    int32_t D_per_dim, dt_softplus;
    int32_t return_all;   // states[c] for every chunk instead of states[b] per request
};

// ------------------------------------------------------------------ types

template <typename T> struct Mfma;

template <>
struct Mfma<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x4 mma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x16 mma32(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x4 mma16(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x16 mma32(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// A 16-bit operand of the matrix cores that stands for an fp32 value v is the
// pair hi = io(v), lo = io(v - hi): the two products hi * b + lo * b, summed in
// fp32, carry v to about 2^-16 (bf16) or 2^-22 (fp16) of itself instead of the
// 2^-9 / 2^-12 of one rounding. The scan feeds its decayed C B^T entries and
// the entering states this way, the walk its weighted x; x, B and C are exact
// in the io type and go in whole. (The per-chunk C B^T entries are kept in
// fp32 for the same reason.)
template <typename IT>
__device__ __forceinline__ void split16(float v, IT& hi, IT& lo) {
    hi = static_cast<IT>(v);
    lo = static_cast<IT>(v - static_cast<float>(hi));
}

// Each chunk's entering state crosses memory from the walk to the scan as, per
// (chunk, head), the high parts hi = io(v) of its P x N elements, then their
// low parts as signed bytes q = round((v - hi) / u), u = ulp(hi) / 256, clamped
// to +-127: three bytes per element instead of the four of two io-type planes.
// q u is exact in the io type (at most 7 significant bits), so the scan feeds
// hi and q u to the matrix cores as the pair above; |v - hi - q u| <= u / 2
// (u with the clamp, when |v - hi| is exactly ulp(hi) / 2), i.e. 2^-16 (bf16)
// or 2^-19 (fp16) of |hi|. u is taken from hi's fp32 exponent field, the same
// on both sides.
constexpr int kEnterBytes = 3;
template <typename T> struct IoMantissa;
template <> struct IoMantissa<__bf16> { static constexpr int bits = 7; };
template <> struct IoMantissa<_Float16> { static constexpr int bits = 10; };
template <typename IT>
__device__ __forceinline__ int low_unit_exp(float hi) {
    return static_cast<int>((__float_as_uint(hi) >> 23) & 0xFFu) - 127 - IoMantissa<IT>::bits - 8;
}
// The low byte of v given its high part (as an fp32 value).
template <typename IT>
__device__ __forceinline__ unsigned low_byte(float v, float hi) {
    const float q = __builtin_rintf(__builtin_amdgcn_ldexpf(v - hi, -low_unit_exp<IT>(hi)));
    return static_cast<unsigned>(static_cast<int>(fminf(fmaxf(q, -127.f), 127.f))) & 0xFFu;
}
// The low part q u back from the byte q (sign-extended) and the high part.
template <typename IT>
__device__ __forceinline__ float low_value(float hi, int q) {
    return __builtin_amdgcn_ldexpf(static_cast<float>(q), low_unit_exp<IT>(hi));
}
// Headdim columns one walk item or one scan workgroup covers; headdim is a
// multiple of it.
constexpr int kHeadBlock = 64;
// Largest dstate block of one walk item.
constexpr int kWalkStateBlock = 128;

// 16-bit io value <-> bits <-> fp32.
template <typename T>
__device__ __forceinline__ float f32_of(unsigned short b) {
    return static_cast<float>(__builtin_bit_cast(T, b));
}
template <typename T>
__device__ __forceinline__ unsigned short bits_of(float v) {
    return __builtin_bit_cast(unsigned short, static_cast<T>(v));
}

// Streaming data (x, z, out) is read and written non-temporally (bload_nt and
// non-temporal stores), so that it does not push the operands every head of a
// group shares (B, C, C B^T of the chunk) out of L2.

// Raw buffer over `bytes` bytes from `base` (dword 3 of a gfx9 raw buffer:
// 32-bit data format, no swizzle). A load at an offset at or past `bytes`
// returns zeros without a memory access; `bytes` 0 makes every load zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             0x00020000);
}
// An offset no range reaches (ranges stay below 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Sixteen bytes, cached normally / non-temporally (cache-policy bit NT).
__device__ __forceinline__ u16x8 bload(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u16x8 bload_nt(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ float bload_f32(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Four consecutive state-type elements at byte offset `off` of a buffer
// descriptor, as fp32 (one 16-byte load for fp32, one 8-byte load otherwise),
// and back.
// `soff` is a wave-uniform part of the offset (it travels in a scalar register).
template <typename ST>
__device__ __forceinline__ f32x4 bload_state4(Rsrc r, uint32_t off, uint32_t soff) {
    if constexpr (sizeof(ST) == 4) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
    } else {
        typedef ST st4 __attribute__((ext_vector_type(4)));
        const st4 v = __builtin_bit_cast(st4, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
        return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                     static_cast<float>(v[3])};
    }
}
template <typename ST>
__device__ __forceinline__ void bstore_state4(Rsrc r, uint32_t off, uint32_t soff, f32x4 v) {
    typedef ST st4 __attribute__((ext_vector_type(4)));
    st4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<ST>(v[i]);
    if constexpr (sizeof(ST) == 4) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), r, off, soff, 0);
    } else {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), r, off, soff, 0);
    }
}

// softplus(v) = max(v, 0) + log1p(exp(-|v|)) with the hardware exp2, log2 and
// reciprocal; log1p(e) as log(u) e / (u - 1), u = 1 + e rounded, which cancels
// the rounding of u (a few ulp of fp32 in all).
__device__ __forceinline__ float softplus_fast(float v) {
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(v));
    const float u = 1.f + e;
    const float l = u == 1.f ? e : 0.6931471805599453f * __builtin_amdgcn_logf(u) * e *
                                       __builtin_amdgcn_rcpf(u - 1.f);
    return fmaxf(v, 0.f) + l;
}

// The gate z sigmoid(z) with the hardware exp2 and reciprocal (about 2 ulp of
// fp32, far below the 16-bit rounding of the result).
__device__ __forceinline__ float gate_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// A value every lane of the wave reads at one address, through the scalar data
// cache (read only). Only for workspace and metadata an earlier launch wrote:
// the constant address space tells the compiler nothing in this launch stores
// there, which lets it use a scalar load instead of a vector one whose wait
// would also cover every vector load issued before it.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)(ptr);
}

// A chunk's descriptor, all 16 bytes in one scalar load.
__device__ __forceinline__ ChunkDesc load_desc(const SsdParams& p, int64_t c) {
    static_assert(sizeof(ChunkDesc) == sizeof(u32x4), "one 16-byte load");
    return __builtin_bit_cast(ChunkDesc, ld_uniform(reinterpret_cast<const u32x4*>(p.desc + c)));
}

// Workgroups are dealt round robin to the XCDs, each with its own L2. Renumber
// them so that each XCD walks a contiguous range of chunk-major tiles: all heads
// of a chunk then meet the chunk's shared operands in one L2.
__device__ __forceinline__ int64_t xcd_order(int64_t id, int64_t n) { return ssu::xcd_tile(id, n); }

// Entry i of a chunk-metadata array (the caller's, read only), one value for
// the whole wave.
__device__ __forceinline__ int64_t meta_uniform(const void* ptr, int is64, int64_t i) {
    return is64 ? ld_uniform(static_cast<const int64_t*>(ptr) + i)
                : static_cast<int64_t>(ld_uniform(static_cast<const int32_t*>(ptr) + i));
}

// Chunk c's first token and length from the caller's cu_chunk_seqlens (read by
// prep, which hands them on in the chunk descriptor, and by bmm); a range
// outside [0, tokens], running backwards or longer than Q counts as empty.
struct Chunk {
    int64_t lo;
    int len;
};

template <int Q>
__device__ __forceinline__ Chunk chunk_of(const SsdParams& p, int64_t c) {
    const int64_t lo = meta_uniform(p.cu_chunk, p.meta_i64, c);
    const int64_t hi = meta_uniform(p.cu_chunk, p.meta_i64, c + 1);
    if (lo < 0 || hi < lo || hi > p.tokens || hi - lo > Q) return {0, 0};
    return {lo, static_cast<int>(hi - lo)};
}

// ------------------------------------------------------------ request list

// One workgroup of the front launch:
//  - list_head[c] / list_next[b]: the requests b whose last chunk index is c, as
//    a linked list per chunk (order unspecified; each b appears once), when final
//    states are returned per request;
//  - the runs: maximal ranges of chunks each continuing the one before (a run
//    starts at every chunk that opens a request: the first chunk, and every
//    chunk whose seq_idx differs from the previous chunk's), as (first chunk,
//    length) sorted by length, longest first (up to kSortRuns runs; more stay in
//    chunk order), for the state walk.
// It reads only the caller's metadata, so it needs nothing from prep.
constexpr int kListThreads = kThreads;
constexpr int kSortRuns = 2048;

__device__ void list_body(const SsdParams& p) {
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    constexpr int NW = kListThreads / 64;
    if (!p.return_all && p.batch > 0) {
        for (int64_t c = tid; c < p.nchunks; c += kListThreads) p.list_head[c] = -1;
        __syncthreads();
        for (int64_t b = tid; b < p.batch; b += kListThreads) {
            const int64_t c = load_index(p.lci, p.meta_i64, b);
            if (c >= 0 && c < p.nchunks) p.list_next[b] = atomicExch(&p.list_head[c], static_cast<int>(b));
        }
    }
    // Run starts, compacted in chunk order.
    __shared__ int s_count[NW];
    int base = 0;
    for (int64_t c0 = 0; c0 < p.nchunks; c0 += kListThreads) {
        const int64_t c = c0 + tid;
        const bool start = c < p.nchunks &&
                           (c == 0 || load_index(p.seq_idx, p.meta_i64, c) !=
                                          load_index(p.seq_idx, p.meta_i64, c - 1));
        const unsigned long long m = __ballot(start);
        if (lane == 0) s_count[wave] = __popcll(m);
        __syncthreads();
        int off = base, total = 0;
        for (int w = 0; w < NW; ++w) {
            off += w < wave ? s_count[w] : 0;
            total += s_count[w];
        }
        if (start) p.run_first[off + __popcll(m & ((1ull << lane) - 1))] = static_cast<int>(c);
        __syncthreads();
        base += total;
    }
    const int nruns = base;
    // Lengths, then each run's rank among them (longest first, ties in chunk order).
    for (int r = tid; r < nruns; r += kListThreads) {
        const int first = p.run_first[r];
        const int len = (r + 1 < nruns ? p.run_first[r + 1] : static_cast<int>(p.nchunks)) - first;
        p.walk_len[r] = len;  // by run, until ranked below
    }
    __syncthreads();
    int first[kSortRuns / kListThreads], len[kSortRuns / kListThreads], rank[kSortRuns / kListThreads];
    const bool sort = nruns <= kSortRuns;
#pragma unroll
    for (int i = 0; i < kSortRuns / kListThreads; ++i) {
        const int r = tid + i * kListThreads;
        if (!sort || r >= nruns) continue;
        first[i] = p.run_first[r];
        len[i] = p.walk_len[r];
        int k = 0;
        for (int j = 0; j < nruns; ++j) {
            const int lj = p.walk_len[j];
            k += lj > len[i] || (lj == len[i] && j < r);
        }
        rank[i] = k;
    }
    __syncthreads();  // every length is read before the ranked order overwrites it
    if (sort) {
#pragma unroll
        for (int i = 0; i < kSortRuns / kListThreads; ++i) {
            const int r = tid + i * kListThreads;
            if (r >= nruns) continue;
            p.walk_first[rank[i]] = first[i];
            p.walk_len[rank[i]] = len[i];
        }
    } else {
        for (int r = tid; r < nruns; r += kListThreads) p.walk_first[r] = p.run_first[r];
    }
    if (tid == 0) p.walk_info[0] = nruns;
}

// -------------------------------------------------------------------- prep

// One wave per (chunk, head): the clamped steps v_s and the running sums
// cum_s = sum_{j<=s} A v_j (fp64) of the chunk, handed on as the chunk-state
// weights w = exp(cum_last - cum_s) v_s, the scan's decay exponents with the
// step folded in, cum_s log2(e) - log2(v_s) (+inf for a zero step), and
// cum_s log2(e), and
// cum_last; zero steps and weights past the chunk's end. The wave of head 0
// writes the chunk's descriptor. Lane l owns tokens l + 64 r. Workgroup `id` of
// `count` (chunk x groups of four heads).
constexpr int kPrepThreads = kThreads;

__host__ __device__ constexpr int64_t prep_blocks(int64_t nchunks, int64_t nheads) {
    return nchunks * ((nheads + kPrepThreads / 64 - 1) / (kPrepThreads / 64));
}

template <int Q>
__device__ void prep_body(const SsdParams& p, int64_t id, int64_t count) {
    constexpr int R = Q / 64;
    constexpr int HW = kPrepThreads / 64;  // heads per workgroup
    constexpr float kLog2e = 1.4426950408889634f;
    const int H = p.nheads;
    const int hq = (H + HW - 1) / HW;
    // XCD-contiguous numbering: the workgroups of a chunk share its dt rows in one L2.
    const int64_t wg = xcd_order(id, count);
    const int64_t c = wg / hq;
    const int h = static_cast<int>(wg % hq) * HW + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    if (h >= H) return;
    const Chunk ch = chunk_of<Q>(p, c);
    if (h == 0 && lane == 0) {
        const int64_t req = meta_uniform(p.seq_idx, p.meta_i64, c);
        const bool opens = c == 0 || req != meta_uniform(p.seq_idx, p.meta_i64, c - 1);
        int32_t enter = kEnterCarry;
        if (opens) enter = p.init && req >= 0 && req < p.batch ? static_cast<int32_t>(req) : kEnterZero;
        p.desc[c] = ChunkDesc{ch.lo, ch.len, enter};
    }
    float u[R];
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = 0.f;
    if (ch.len > 0) {
        // One branch on the dt type around all loads, so they are issued together.
        int64_t idx[R];
#pragma unroll
        for (int r = 0; r < R; ++r) idx[r] = (ch.lo + min(64 * r + lane, ch.len - 1)) * H + h;
        if (p.dt_dtype == kF32) {
#pragma unroll
            for (int r = 0; r < R; ++r) u[r] = static_cast<const float*>(p.dt)[idx[r]];
        } else if (p.dt_dtype == kF16) {
#pragma unroll
            for (int r = 0; r < R; ++r) u[r] = static_cast<float>(static_cast<const _Float16*>(p.dt)[idx[r]]);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) u[r] = static_cast<float>(static_cast<const __bf16*>(p.dt)[idx[r]]);
        }
    }
    const double A = static_cast<double>(ld_uniform(p.A + h));
    float v[R];
    double cum[R];
    double carry = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = 64 * r + lane;
        float x = u[r];
        if (p.dt_bias) x += ld_uniform(p.dt_bias + h);
        if (p.dt_softplus) x = softplus_fast(x);
        x = fminf(fmaxf(x, p.dt_min), p.dt_max);
        v[r] = s < ch.len ? x : 0.f;
        double a = A * static_cast<double>(v[r]);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_up(a, d);
            if (lane >= d) a += o;
        }
        cum[r] = a + carry;
        carry = __shfl(cum[r], 63);
    }
    const int64_t base = (c * H + h) * Q;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int s = 64 * r + lane;
        p.w[base + s] = s < ch.len ? expf(static_cast<float>(carry - cum[r])) * v[r] : 0.f;
        const float c2 = static_cast<float>(cum[r]) * kLog2e;
        p.cv[2 * base + s] = c2 - __builtin_amdgcn_logf(v[r]);
        p.cv[2 * base + Q + s] = c2;
    }
    if (lane == 0) p.cumlast[c * H + h] = static_cast<float>(carry);
}

// --------------------------------------------------------------------- bmm

// CB[c, g] = C B^T over the chunk's tokens, lower triangle of 32x32 tiles
// (s <= t needs no more): one wave per tile, 32x32x16 MFMA with both operands
// straight from memory (eight consecutive dstate values per lane are
// contiguous), every operand load issued before the first product. Rows past
// the chunk's length read its last token and are never used. The chunk's token
// range comes from the caller's cu_chunk_seqlens, so this needs nothing from
// prep. Workgroup `id` of `count` (chunk x group x tile blocks).
template <int Q> __host__ __device__ constexpr int bmm_tiles() { return (Q / 32) * (Q / 32 + 1) / 2; }
template <int Q> __host__ __device__ constexpr int bmm_blocks() { return (bmm_tiles<Q>() + kWaves - 1) / kWaves; }

template <typename IT, int N, int Q>
__device__ void bmm_body(const SsdParams& p, int64_t id, int64_t count) {
    typedef typename Mfma<IT>::v8 v8;
    // XCD-contiguous numbering: the workgroups of a (chunk, group) share its C and
    // B rows in one L2.
    const int64_t wg = xcd_order(id, count);
    const int64_t cg = wg / bmm_blocks<Q>();
    const int tile = static_cast<int>(wg % bmm_blocks<Q>()) * kWaves +
                     __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    if (tile >= bmm_tiles<Q>()) return;
    const int64_t c = cg / p.ngroups;
    const int g = static_cast<int>(cg % p.ngroups);
    const Chunk d = chunk_of<Q>(p, c);
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    const int sj = tile - ti * (ti + 1) / 2;
    if (ti * 32 >= d.len) return;
    const int lane = threadIdx.x % 64;
    const IT* Cp = static_cast<const IT*>(p.C);
    const IT* Bp = static_cast<const IT*>(p.B);
    const int t = min(ti * 32 + lane % 32, d.len - 1);
    const int s = min(sj * 32 + lane % 32, d.len - 1);
    const v8* ca = reinterpret_cast<const v8*>(Cp + ((d.lo + t) * p.ngroups + g) * N);
    const v8* bb = reinterpret_cast<const v8*>(Bp + ((d.lo + s) * p.ngroups + g) * N);
    v8 ra[N / 16], rb[N / 16];
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
        ra[k] = ca[2 * k + lane / 32];
        rb[k] = bb[2 * k + lane / 32];
    }
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < N / 16; ++k) acc = Mfma<IT>::mma32(ra[k], rb[k], acc);
    float* out = p.cb + (c * p.ngroups + g) * Q * Q;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = ti * 32 + 8 * (i / 4) + 4 * (lane / 32) + i % 4;
        out[row * Q + sj * 32 + lane % 32] = acc[i];
    }
}

// ------------------------------------------------------------------ front

// The three short stages before the state walk share one launch: none reads
// what another writes (each derives chunk ranges and request openings from the
// caller's metadata), and the walk and the scan, which read all three, come in
// later launches. Workgroup ranges, each starting at a multiple of the XCD
// count so that the XCD-contiguous numbering inside a range holds: the list
// (first, so that its serial work starts at once; the other workgroups of its
// range return at once), then prep, then the C B^T tiles.
__host__ __device__ constexpr int64_t round_to_xcds(int64_t n) {
    return (n + ssu::kXcds - 1) / ssu::kXcds * ssu::kXcds;
}

template <int Q>
__host__ __device__ constexpr int64_t front_blocks(int64_t nchunks, int64_t nheads, int64_t ngroups) {
    return ssu::kXcds + round_to_xcds(prep_blocks(nchunks, nheads)) + nchunks * ngroups * bmm_blocks<Q>();
}

template <typename IT, int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_front_kernel(const SsdParams p) {
    int64_t b = blockIdx.x;
    if (b < ssu::kXcds) {
        if (b == 0) list_body(p);
        return;
    }
    b -= ssu::kXcds;
    const int64_t np = prep_blocks(p.nchunks, p.nheads);
    if (b < round_to_xcds(np)) {
        if (b < np) prep_body<Q>(p, b, np);
        return;
    }
    b -= round_to_xcds(np);
    bmm_body<IT, N, Q>(p, b, p.nchunks * p.ngroups * bmm_blocks<Q>());
}

// ----------------------------------------------------------- LDS layout

// Transposed tiles in LDS keep the 16-byte chunks of each row permuted by the
// row's octet: chunk c of row r lives at chunk c ^ ((r / 8) % 8). The
// transposing stores (eight rows at once) then spread over the banks, and a
// fragment read (eight consecutive values of one row) stays one 16-byte access.
// Rows hold a multiple of 64 elements, so the permutation stays inside the row.
__device__ __forceinline__ int swz(int r, int col) {
    return (((col >> 3) ^ ((r >> 3) & 7)) << 3) | (col & 7);
}

// -------------------------------------------------------------- state walk

// One work item per (run, head): the head's state S (P x N, fp32) walks the
// run's chunks in order, S = exp(cum_last) S + sum_s w_s x_s B_s^T, held as S^T
// in the matrix-core accumulators (wave w owns dstate rows [32 (w / 2), +32)
// and headdim columns [32 (w % 2), +32) of S^T). A chunk's tokens are staged in
// blocks of KB: B^T [N][KB] and the weighted x^T [P][KB] as high and low 16-bit
// parts; the next block's operands are requested before the current block's
// products. After each chunk the state leaves as the next chunk's entering
// state (high parts and low bytes, for the scan) and in the state type where
// it is returned. The run's entering state is the request's initial state (also
// handed to the scan that way) or zeros. Workgroup i takes items i, i + grid, ...; the items come
// longest run first, so the long walks start at once.
constexpr int kWalkKB = 128;
constexpr int kWalkPitch = kWalkKB + 8;
__host__ __device__ constexpr int walk_threads(int N) { return 4 * N; }
__host__ __device__ constexpr unsigned walk_lds_bytes(int P, int N) {
    return 2u * (N + 2 * P) * kWalkPitch;
}

template <typename IT, typename ST, int N, int Q>
__global__ __launch_bounds__(walk_threads(N), N == 128 ? 4 : 2) void ssd_state_walk_kernel(const SsdParams p) {
    // N is the dstate block of one item (the whole dstate up to 128, else 128 of
    // it) and P = kHeadBlock the headdim block: the state's (p, n) entries evolve
    // independently, so a head's state splits into blocks walked as items of
    // their own. PF and NF are the full headdim and dstate (row strides).
    constexpr int P = kHeadBlock;
    typedef typename Mfma<IT>::v8 v8;
    constexpr int NT = walk_threads(N), NW = NT / 64;
    constexpr int KB = Q < kWalkKB ? Q : kWalkKB, XP = kWalkPitch;
    constexpr int NSB = Q / KB;                          // blocks per chunk
    static_assert(NW == 2 * (N / 32), "waves: dstate row blocks x headdim halves");
    constexpr int XQ = P / 8, BQ = N / 8;                // 16-byte pieces of a token's x / B row
    constexpr int XN = (KB / 2) * XQ, BN = (KB / 2) * BQ;  // two-token pieces per block
    constexpr int XPASS = XN / NT, BPASS = BN / NT;
    static_assert(XPASS * NT == XN && BPASS * NT == BN, "whole passes");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int n0 = 32 * (wave / 2), q0 = 32 * (wave % 2);

    extern __shared__ __align__(16) unsigned char smem[];
    unsigned short* bt = reinterpret_cast<unsigned short*>(smem);  // [N][XP]
    unsigned short* xhi = bt + N * XP;                             // [P][XP]
    unsigned short* xlo = xhi + P * XP;

    const int H = p.nheads, PF = p.headdim, NF = p.dstate;
    const int PB = PF / P, NB = NF / N;                  // headdim and dstate blocks
    const int SB = PB * NB;                              // items per (run, head)
    const int64_t nitems = static_cast<int64_t>(ld_uniform(p.walk_info)) * H * SB;
    const uint32_t xrow = static_cast<uint32_t>(H * PF * 2), brow = static_cast<uint32_t>(p.ngroups * NF * 2);
    const int64_t tile = static_cast<int64_t>(H) * PF * NF;
    const bool lists = !p.return_all && p.batch > 0;
    // First byte of chunk c's entering state for head h (high parts, then low bytes).
    auto enter_tile = [&](int64_t c, int h) { return (c * H + h) * (kEnterBytes * static_cast<int64_t>(PF) * NF); };

    // Workgroups are dealt to the XCDs round robin, so with a grid of a multiple
    // of the XCD count each XCD always sees the same residue of item % XCDs.
    // Heads are permuted so that residue x means the contiguous heads
    // [x H / XCDs, (x + 1) H / XCDs): every XCD works on every run, and the
    // heads sharing B rows (a group, or part of one) share one L2.
    const bool by_xcd = (H * SB) % ssu::kXcds == 0 && gridDim.x % ssu::kXcds == 0;
    // Items are dealt in rounds of one per workgroup, every other round in
    // reverse ("snake" order): with the runs longest first, a workgroup that
    // got one of the longest walks gets one of the shortest next.
    const int64_t G = gridDim.x;
    for (int64_t round = 0;; ++round) {
        const int64_t item = round * G + ((round & 1) ? G - 1 - blockIdx.x : blockIdx.x);
        if (item >= nitems) {
            if (round * G >= nitems) break;
            continue;  // this round's tail is short; a reversed round may still hold an item
        }
        // (run, head, block) with the H * SB (head, block) pairs as "virtual heads"
        // permuted like the heads above: an XCD's share is whole heads.
        const int HS = H * SB;
        const int r = static_cast<int>(item / HS), u = static_cast<int>(item % HS);
        const int vh = by_xcd ? (u % ssu::kXcds) * (HS / ssu::kXcds) + u / ssu::kXcds : u;
        const int h = vh / SB, pb = (vh % SB) / NB, nb = vh % NB;
        const int c0 = ld_uniform(p.walk_first + r), nc = ld_uniform(p.walk_len + r);
        const int g = h / p.heads_per_group;
        const IT* xh = static_cast<const IT*>(p.x) + h * PF + pb * P;
        const IT* bg = static_cast<const IT*>(p.B) + g * NF + nb * N;
        // This item's block of the head's [PF][NF] state: rows pb P.., columns nb N..
        const int64_t hs = static_cast<int64_t>(h) * PF * NF + static_cast<int64_t>(pb) * P * NF + nb * N;
        // Bytes from the block's first element to past its last, rows NF apart.
        auto block_bytes = [&](int esz) { return static_cast<uint32_t>(((P - 1) * NF + N) * esz); };
        // Offset of this lane's four consecutive state elements of tile (nt, qt)
        // inside the block: a per-lane part and a wave-uniform part per tile.
        const uint32_t lane_el = static_cast<uint32_t>((q0 + lane % 16) * NF + n0 + 4 * (lane / 16));
        auto tile_el = [&](int nt, int qt) { return static_cast<uint32_t>(16 * qt * NF + 16 * nt); };

        // The operands of one block: x and B rows of tokens [s0, s0 + KB) of chunk c
        // (zeros past its end) and the weights of the token pairs.
        u16x8 rx[XPASS][2], rb[BPASS][2];
        float2 rw[XPASS];
        auto fetch = [&](const ChunkDesc& d, int c, int s0) {
            const Rsrc xr = make_rsrc(xh + d.lo * H * PF, d.len * xrow);
            const Rsrc br = make_rsrc(bg + d.lo * p.ngroups * NF, d.len * brow);
            const Rsrc wr = make_rsrc(p.w + (static_cast<int64_t>(c) * H + h) * Q, 4u * Q);
#pragma unroll
            for (int i = 0; i < XPASS; ++i) {
                const int idx = tid + NT * i, q = idx % XQ, s = s0 + 2 * (idx / XQ);
                const uint32_t off = s * xrow + 16 * q;
                rx[i][0] = bload_nt(xr, off);
                rx[i][1] = bload_nt(xr, off + xrow);
                rw[i] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(wr, 4u * s, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < BPASS; ++i) {
                const int idx = tid + NT * i, q = idx % BQ, s = s0 + 2 * (idx / BQ);
                const uint32_t off = s * brow + 16 * q;
                rb[i][0] = bload(br, off);
                rb[i][1] = bload(br, off + brow);
            }
        };

        ChunkDesc d = load_desc(p, c0);
        fetch(d, c0, 0);
        f32x4 acc[2][2];
        const bool init = d.enter >= 0 && d.enter < p.batch;
        if (init) {
            const Rsrc ir = make_rsrc(static_cast<const ST*>(p.init) + d.enter * tile + hs,
                                      block_bytes(sizeof(ST)));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    acc[nt][qt] = bload_state4<ST>(ir, sizeof(ST) * lane_el, sizeof(ST) * tile_el(nt, qt));
        } else {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) acc[nt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        // The state as chunk c's entering state: the high parts and the low bytes
        // of this item's block (rows NF apart in the head's [PF][NF] tile of
        // each), through the B^T area of LDS so that every store writes whole
        // 16-byte pieces of whole rows: each wave drops its part of S^T into LDS
        // (16-byte chunks of row p permuted by p, which spreads the writes of
        // sixteen rows over the banks), then the workgroup copies the rows out.
        // The caller makes sure every wave is done with the B^T area; the next
        // use of LDS is behind a barrier.
        auto store_enter = [&](int64_t c) {
            const Rsrc er = make_rsrc(static_cast<unsigned char*>(p.s16) + enter_tile(c, h),
                                      static_cast<uint32_t>(kEnterBytes * PF * NF));
            const uint32_t blk = static_cast<uint32_t>(pb * P * NF + nb * N);  // block's first element
            typedef unsigned short t4 __attribute__((ext_vector_type(4)));
            constexpr int CPR = N * 2 / 16;  // 16-byte chunks per row: high parts
            constexpr int CPL = N / 16;      // low bytes
            constexpr unsigned HI = P * N * 2;  // LDS bytes of the high parts
            static_assert(HI + P * N <= 2u * N * XP, "both parts fit the B^T area");
            unsigned char* lt = reinterpret_cast<unsigned char*>(bt);
            // High parts first, then the low bytes (the high part recomputed), which
            // keeps few values live beside the next block's operands.
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int pr = q0 + 16 * qt + lane % 16, n = n0 + 16 * nt + 4 * (lane / 16);
                    const int byte = n * 2;
                    t4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = bits_of<IT>(acc[nt][qt][i]);
                    *reinterpret_cast<t4*>(lt + pr * N * 2 + (((byte / 16) ^ (pr % CPR)) * 16) + byte % 16) = v;
                }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int pr = q0 + 16 * qt + lane % 16, n = n0 + 16 * nt + 4 * (lane / 16);
                    unsigned lo = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        lo |= low_byte<IT>(acc[nt][qt][i], f32_of<IT>(bits_of<IT>(acc[nt][qt][i]))) << (8 * i);
                    *reinterpret_cast<unsigned*>(lt + HI + pr * N + (((n / 16) ^ (pr % CPL)) * 16) + n % 16) = lo;
                }
            lds_barrier();
            constexpr int HP = P * CPR / NT, LP = P * CPL / NT;  // pieces per thread
            static_assert(HP * NT == P * CPR && LP * NT == P * CPL, "whole pieces");
            // One piece at a time, which bounds the registers the copy holds: the
            // high parts' pieces, then the low bytes'.
#pragma unroll 1
            for (int i = 0; i < HP + LP; ++i) {
                const bool high = i < HP;
                const int idx = tid + NT * (high ? i : i - HP);
                const int cpr = high ? CPR : CPL, pr = idx / cpr, ch = idx % cpr;
                const u32x4 v = *reinterpret_cast<const u32x4*>(
                    lt + (high ? pr * N * 2 : HI + pr * N) + ((ch ^ (pr % cpr)) * 16));
                __builtin_amdgcn_raw_buffer_store_b128(v, er, (blk + pr * NF) * (high ? 2 : 1) + ch * 16,
                                                       high ? 0u : static_cast<uint32_t>(2 * PF * NF), 0);
            }
        };
        // The run's initial state is the first chunk's entering state too (LDS
        // is free: the previous item ended with a barrier, and the first block
        // stages behind one).
        if (init) store_enter(c0);

        // The returned states, written from the accumulators directly (each
        // chunk's with return_intermediate_states, else only the requests'
        // last chunks').
        auto put = [&](int64_t row) {
            const Rsrc sr = make_rsrc(static_cast<ST*>(p.states) + row * tile + hs, block_bytes(sizeof(ST)));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    bstore_state4<ST>(sr, sizeof(ST) * lane_el, sizeof(ST) * tile_el(nt, qt), acc[nt][qt]);
        };

        // Per-chunk scalars are requested a chunk ahead of their use.
        ChunkDesc dn = load_desc(p, (nc > 1 ? c0 + 1 : c0));
        float cl = ld_uniform(p.cumlast + static_cast<int64_t>(c0) * H + h);
        int rq = lists ? ld_uniform(p.list_head + c0) : -1;
        for (int k = 0; k < nc; ++k) {
            const int c = c0 + k;
            const bool more = k + 1 < nc;
            const ChunkDesc dnn = load_desc(p, (k + 2 < nc ? c + 2 : c));
            const float cln = ld_uniform(p.cumlast + static_cast<int64_t>(more ? c + 1 : c) * H + h);
            const int rqn = lists ? ld_uniform(p.list_head + (more ? c + 1 : c)) : -1;
            const float decay = expf(cl);
            const int first_req = rq;

#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int s0 = KB * sb;
                lds_barrier();  // the previous block's products are done with LDS
#pragma unroll
                for (int i = 0; i < BPASS; ++i) {
                    const int idx = tid + NT * i, q = idx % BQ, j = 2 * (idx / BQ);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = 8 * q + e;
                        *reinterpret_cast<unsigned*>(bt + row * XP + swz(row, j)) =
                            rb[i][0][e] | (static_cast<unsigned>(rb[i][1][e]) << 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < XPASS; ++i) {
                    const int idx = tid + NT * i, q = idx % XQ, j = 2 * (idx / XQ);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float a0 = f32_of<IT>(rx[i][0][e]) * rw[i].x;
                        const float a1 = f32_of<IT>(rx[i][1][e]) * rw[i].y;
                        const unsigned short hi0 = bits_of<IT>(a0), hi1 = bits_of<IT>(a1);
                        const unsigned short lo0 = bits_of<IT>(a0 - f32_of<IT>(hi0));
                        const unsigned short lo1 = bits_of<IT>(a1 - f32_of<IT>(hi1));
                        const int row = 8 * q + e, o = row * XP + swz(row, j);
                        *reinterpret_cast<unsigned*>(xhi + o) = hi0 | (static_cast<unsigned>(hi1) << 16);
                        *reinterpret_cast<unsigned*>(xlo + o) = lo0 | (static_cast<unsigned>(lo1) << 16);
                    }
                }
                if (sb == 0) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[nt][qt][i] *= decay;
                }
                // The next block's operands: this chunk's next block, else the next
                // chunk's first (none past the run: an empty range loads zeros).
                if (sb + 1 < NSB)
                    fetch(d, c, s0 + KB);
                else
                    fetch(more ? dn : ChunkDesc{0, 0, 0}, more ? c + 1 : c, 0);
                lds_barrier();
#pragma unroll
                for (int kk = 0; kk < KB; kk += 32) {
                    if (s0 + kk >= d.len) break;
                    const int col = kk + 8 * (lane / 16);
                    v8 a[2], xf[2][2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int row = n0 + 16 * nt + lane % 16;
                        a[nt] = *reinterpret_cast<const v8*>(bt + row * XP + swz(row, col));
                    }
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        const int row = q0 + 16 * qt + lane % 16, o = row * XP + swz(row, col);
                        xf[qt][0] = *reinterpret_cast<const v8*>(xhi + o);
                        xf[qt][1] = *reinterpret_cast<const v8*>(xlo + o);
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int qt = 0; qt < 2; ++qt) {
                            acc[nt][qt] = Mfma<IT>::mma16(a[nt], xf[qt][0], acc[nt][qt]);
                            acc[nt][qt] = Mfma<IT>::mma16(a[nt], xf[qt][1], acc[nt][qt]);
                        }
                }
            }
            // The state after chunk c: the next chunk's entering state if the run
            // goes on, and the returned states (state type).
            if (more) {
                lds_barrier();  // every wave is done with this block's operands
                store_enter(c + 1);
            }
            if (p.return_all) {
                put(c);
            } else {
                int b = first_req;
                for (int64_t guard = 0; guard < p.batch && b >= 0 && b < p.batch; ++guard) {
                    put(b);
                    b = ld_uniform(p.list_next + b);
                }
            }
            d = dn;
            dn = dnn;
            cl = cln;
            rq = rqn;
        }
        __syncthreads();  // every wave is done with LDS before the next item stages
    }
}

// -------------------------------------------------------------------- scan

// The scan runs Q / 32 waves: two 16-token tiles of the chunk per wave.
__host__ __device__ constexpr int scan_threads(int Q) { return 2 * Q; }
constexpr int scan_pitch(int Q) { return Q + 8; }       // (v x)^T row pitch, elements
constexpr int state_pitch(int N) { return N + 8; }      // entering-state row pitch

// LDS bytes of the scan kernel: the decay exponents with the steps folded in
// and the log2-scaled running sums (fp32), the skip coefficients, the entering
// state's two planes [2][P][N + 8] and x^T [P][Q + 8], all three in the io type.
// The epilogue's fp32 scratch (16 rows per wave) then takes the x^T area and
// what follows it.
__host__ __device__ constexpr int scan_epilogue_pitch(int P) { return P + 4; }
// Waves per SIMD the scan is compiled for (its register budget): four for
// chunks of 256 (two 8-wave workgroups per CU, as many as its LDS allows at
// dstate 128), three for chunks of 128 (three 4-wave workgroups at dstate 128;
// its two tiles of C B^T in flight need more than 128 registers). At dstate 256
// the entering state's planes leave LDS room for one workgroup per CU: two
// waves per SIMD for chunks of 256, one for chunks of 128.
__host__ __device__ constexpr int scan_waves_per_simd(int N, int Q) {
    return N >= 256 ? (Q >= 256 ? 2 : 1) : (Q >= 256 ? 4 : 3);
}
// Blocks of 32 C B^T columns each tile has in flight: one for chunks of 256
// (within 128 registers), two for chunks of 128.
__host__ __device__ constexpr int scan_cb_depth(int Q) { return Q >= 256 ? 1 : 2; }
// The scan holds the entering state in LDS as two io-type planes: the high
// parts and the low parts decoded from their bytes.
constexpr int kScanStatePlanes = 2;
__host__ __device__ constexpr unsigned scan_lds_bytes(int P, int N, int Q) {
    return 4u * Q + 4u * Q + 4u * P + 2u * kScanStatePlanes * P * state_pitch(N) +
           (2u * P * scan_pitch(Q) > 4u * 16 * scan_epilogue_pitch(P) * (scan_threads(Q) / 64)
                ? 2u * P * scan_pitch(Q)
                : 4u * 16 * scan_epilogue_pitch(P) * (scan_threads(Q) / 64));
}

// Heads one scan workgroup takes in turn, the next head's operands loading
// while the current head finishes its epilogue: two for chunks of 128 at dstate
// up to 128 (LDS allows three workgroups per CU there, which leaves registers
// for the loads in flight), else one.
__host__ __device__ constexpr int scan_heads(int N, int Q) { return Q < 256 && N <= 128 ? 2 : 1; }

// x^T and the entering state are stored permuted by swz().

// One workgroup per (chunk, scan_heads consecutive heads, block of kHeadBlock
// headdim columns), the heads one after the other; wave w owns token tiles w
// and 2 NW - 1 - w. The outputs of different headdim columns share nothing but
// the decayed C B^T entries, which each block recomputes. Every load a head
// needs before its first product -- steps, the x tile, the entering state, the
// first C operands, D -- is issued before anything waits (the next head's
// during this head's epilogue), each product's next operands before its
// current matrix-core work.
template <typename IT, typename ST, int N, int Q>
__global__ __launch_bounds__(scan_threads(Q), scan_waves_per_simd(N, Q)) void ssd_scan_kernel(const SsdParams p) {
    constexpr int P = kHeadBlock;
    typedef typename Mfma<IT>::v8 v8;
    constexpr int NT = scan_threads(Q), NW = NT / 64;
    constexpr int PT = P / 16, TT = 2, KN = N / 32;
    constexpr int XP = scan_pitch(Q), SP = state_pitch(N);
    constexpr int XPASS = (Q / 2) * (P / 8) / NT;   // x loads per thread (token pairs x row octets)
    constexpr int SPASS = P * (N / 8) / NT;         // entering-state 16-byte chunks per thread
    static_assert(XPASS * NT == (Q / 2) * (P / 8) && SPASS * NT == P * (N / 8), "passes");
    static_assert((SP * 2) % 16 == 0 && (XP * 2) % 16 == 0, "16-byte rows");

    constexpr int HL = scan_heads(N, Q);
    const int PF = p.headdim, PBK = PF / P;
    const int H = p.nheads, HQ = (H + HL - 1) / HL;
    const int64_t wg = xcd_order(blockIdx.x, gridDim.x);
    const int64_t c = wg / (static_cast<int64_t>(HQ) * PBK);
    const int h0 = static_cast<int>((wg / PBK) % HQ) * HL;
    const int pb = static_cast<int>(wg % PBK);
    const ChunkDesc d = load_desc(p, c);
    if (d.len == 0) return;
    const int len = d.len;
    int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    int lane = tid % 64;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sl = reinterpret_cast<float*>(smem);  // [Q] cum_s log2(e) - log2(v_s)
    float* cum2 = sl + Q;                          // [Q] cum_s log2(e)
    static_assert(NT == 2 * Q, "one value per thread");
    float* sd = cum2 + Q;  // [P] skip coefficients
    unsigned short* sS = reinterpret_cast<unsigned short*>(sd + P);  // [2][P][SP]
    unsigned short* xv = sS + kScanStatePlanes * P * SP;

    const IT* Cp = static_cast<const IT*>(p.C);
    const uint32_t xrow = static_cast<uint32_t>(H * PF * 2);
    // The chunk's first x / z / out row of head h, at this block's columns.
    auto xoff_of = [&](int h) { return (d.lo * H + h) * PF + pb * P; };

    // ---- a head's loads, issued before anything waits: for the first head at
    // the start, for the next one while this one finishes its epilogue.
    const bool has_state = d.enter != kEnterZero;
    const uint32_t sblk = pb * P * N;
    typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
    float step;             // cum_s log2(e) - log2(v_s) (tid < Q), then cum_s log2(e)
    u16x8 rx[XPASS][2];     // x: thread handles row octet q of token pair s
    u16x8 rs[SPASS];        // entering state: high parts of eight elements
    u32x2v rq[SPASS];       // ... and their low bytes
    float dcoef;            // the skip coefficient of headdim row tid (zero without D)
    auto issue = [&](int h) {
        step = p.cv[(c * H + h) * 2 * Q + tid];
        const Rsrc xr = make_rsrc(static_cast<const IT*>(p.x) + xoff_of(h), len * xrow);
#pragma unroll
        for (int r = 0; r < XPASS; ++r) {
            const int idx = tid + NT * r, q = idx % (P / 8), s = 2 * (idx / (P / 8));
            const uint32_t off = s * xrow + 16 * q;
            rx[r][0] = bload_nt(xr, off);
            rx[r][1] = bload_nt(xr, off + xrow);
        }
        // The entering state (zeros for a chunk that opens a request without
        // one): this block's rows (contiguous) of the high parts and of the low
        // bytes, the same eight elements of each per load.
        const Rsrc sr = make_rsrc(static_cast<const unsigned char*>(p.s16) + (c * H + h) * kEnterBytes * PF * N,
                                  has_state ? kEnterBytes * PF * N : 0);
#pragma unroll
        for (int r = 0; r < SPASS; ++r) {
            const uint32_t e = sblk + 8 * (tid + NT * r);
            rs[r] = bload(sr, 2 * e);
            rq[r] = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(sr, e, 2 * PF * N, 0));
        }
        const Rsrc dr = make_rsrc(p.D, p.D ? static_cast<uint32_t>((p.D_per_dim ? H * PF : H) * 4) : 0u);
        dcoef = bload_f32(dr, 4u * (p.D_per_dim ? h * PF + pb * P + min(tid, P - 1) : h));
    };
    issue(h0);
    // Unrolled, so that which copy prefetches is known when compiling: each
    // copy's operand registers are then the only live ones.
#pragma unroll
    for (int j = 0; j < HL; ++j) {
        const int h = h0 + j;
        if (h >= H) break;
        // Each head recomputes its per-lane offsets rather than holding them
        // across the loop (an empty asm makes the lane numbers opaque here).
        asm volatile("" : "+v"(tid), "+v"(lane));
        // C operands of the entering-state product, first k step.
        // Token tiles of this wave: w and 2 NW - 1 - w, so that every wave's pair
        // covers about the same share of the causal triangle (tile i needs i / 2 + 1
        // blocks of C B^T).
        static_assert(TT == 2, "tile pairs");
        int t0_of[TT];
        t0_of[0] = 16 * wave;
        t0_of[1] = 16 * (2 * NW - 1 - wave);
        int trow[TT];
#pragma unroll
        for (int k = 0; k < TT; ++k) trow[k] = min(t0_of[k] + lane % 16, len - 1);
        const int kcol = 8 * (lane / 16);
        bool live[TT];
#pragma unroll
        for (int k = 0; k < TT; ++k) live[k] = t0_of[k] < len;
        const int er = lane / 8, ec = (lane % 8) * (P / 8);
        static_assert(P / 8 == 8, "eight lanes per row, 16 bytes each");
        constexpr int ZL = NW * TT * 2048 <= 2 * kScanStatePlanes * P * SP ? TT : 0;
        u16x8* const zslot = reinterpret_cast<u16x8*>(sS) + 2 * (wave * 64 + lane);  // + 2 * 64 * NW * k

        const int g = h / p.heads_per_group;
        const int64_t xoff = xoff_of(h);
        auto c_frag = [&](int k, int kk) {
            return *reinterpret_cast<const v8*>(Cp + ((d.lo + trow[k]) * p.ngroups + g) * N + kk + kcol);
        };
        v8 cf[TT];
#pragma unroll
        for (int k = 0; k < TT; ++k) cf[k] = c_frag(k, 0);

        // z rows of the epilogue (zeros without z): lane l finishes 8 consecutive
        // columns of rows l / 8 and l / 8 + 8 of each of its tiles, so every store
        // instruction writes eight whole rows. Where every wave's tiles fit the
        // entering-state area they are requested now and parked there once the
        // entering-state product is done with it; otherwise they are requested
        // after the products inside the chunk.
        const Rsrc zr = make_rsrc(p.z ? static_cast<const IT*>(p.z) + xoff : nullptr, p.z ? len * xrow : 0u);
        u16x8 ez[TT][2];
        auto z_load = [&](int k) {
            const uint32_t off = (t0_of[k] + er) * xrow + 2 * ec;
            ez[k][0] = bload_nt(zr, off);
            ez[k][1] = bload_nt(zr, off + 8 * xrow);
        };
#pragma unroll
        for (int k = 0; k < ZL; ++k) z_load(k);

        // Steps, x^T (exact) and the entering state into LDS (after the previous
        // head's epilogue is done with it).
        if (j > 0) lds_barrier();
        sl[tid] = step;  // cum2 follows sl
        if (tid < P) sd[tid] = dcoef;
#pragma unroll
        for (int r = 0; r < XPASS; ++r) {
            const int idx = tid + NT * r, q = idx % (P / 8), s = 2 * (idx / (P / 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pr = 8 * q + e;
                *reinterpret_cast<unsigned*>(xv + pr * XP + swz(pr, s)) =
                    rx[r][0][e] | (static_cast<unsigned>(rx[r][1][e]) << 16);
            }
        }
#pragma unroll
        for (int r = 0; r < SPASS; ++r) {
            const int ci = tid + NT * r, pr = ci / (N / 8), n8 = 8 * (ci % (N / 8));
            u16x8 lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = static_cast<int>(rq[r][e / 4] << (24 - 8 * (e % 4))) >> 24;  // sign-extended byte
                lo[e] = bits_of<IT>(low_value<IT>(f32_of<IT>(rs[r][e]), q));
            }
            *reinterpret_cast<u16x8*>(sS + pr * SP + swz(pr, n8)) = rs[r];
            *reinterpret_cast<u16x8*>(sS + P * SP + pr * SP + swz(pr, n8)) = lo;
        }
        lds_barrier();

        f32x4 acc[TT][PT];
#pragma unroll
        for (int k = 0; k < TT; ++k)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- the entering state: C_t . (S_hi + S_lo), then scaled by exp(cum_t)
        if (has_state) {
#pragma unroll
            for (int ks = 0; ks < KN; ++ks) {
                v8 cn[TT];
                if (ks + 1 < KN) {
#pragma unroll
                    for (int k = 0; k < TT; ++k) cn[k] = c_frag(k, 32 * (ks + 1));
                }
#pragma unroll
                for (int pl = 0; pl < kScanStatePlanes; ++pl) {
                    v8 sf[PT];
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const int pr = 16 * pt + lane % 16;
                        sf[pt] = *reinterpret_cast<const v8*>(sS + pl * P * SP + pr * SP + swz(pr, 32 * ks + kcol));
                    }
#pragma unroll
                    for (int k = 0; k < TT; ++k)
                        if (live[k])
#pragma unroll
                            for (int pt = 0; pt < PT; ++pt) acc[k][pt] = Mfma<IT>::mma16(cf[k], sf[pt], acc[k][pt]);
                }
                if (ks + 1 < KN) {
#pragma unroll
                    for (int k = 0; k < TT; ++k) cf[k] = cn[k];
                }
            }
#pragma unroll
            for (int k = 0; k < TT; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = min(t0_of[k] + 4 * (lane / 16) + i, Q - 1);
                    const float f = __builtin_amdgcn_exp2f(cum2[t]);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[k][pt][i] *= f;
                }
        }

        if constexpr (ZL > 0) {
            lds_barrier();  // every wave is done with the entering state
#pragma unroll
            for (int k = 0; k < ZL; ++k) {
                zslot[2 * 64 * NW * k] = ez[k][0];
                zslot[2 * 64 * NW * k + 1] = ez[k][1];
            }
        }

        // ---- inside the chunk: (C B^T masked, times the decays and the steps v_s)
        // times x. Tile k needs the s blocks kk <= its last row; its C B^T entries
        // are requested two blocks ahead of their products (clamped to the chunk's
        // tile, so a block the tile turns out not to need is a harmless read).
        const float* cbp = p.cb + (c * p.ngroups + g) * Q * Q;
        // Eight fp32 C B^T entries of one row: two 16-byte loads.
        constexpr int CW = 2;
        typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
        constexpr int DEPTH = scan_cb_depth(Q);  // s blocks of C B^T in flight per tile
        u32x4v cb[TT][DEPTH][CW];
        const Rsrc cbr = make_rsrc(cbp, Q * Q * sizeof(float));
        auto cb_load = [&](int k, int kk, int dd) {
            const int t0 = t0_of[k];
            // A block past the tile's last row is never used: its load stays in the
            // instruction stream (the waits count loads) but reads nothing.
            const uint32_t off = kk > t0 + 15 ? kOutOfRange
                                               : ((t0 + lane % 16) * Q + min(kk, Q - 32) + kcol) * sizeof(float);
#pragma unroll
            for (int w = 0; w < CW; ++w)
                cb[k][dd][w] = __builtin_amdgcn_raw_buffer_load_b128(cbr, off + 16 * w, 0, 0);
        };
        auto cb_value = [&](int k, int dd, int j) -> float { return __uint_as_float(cb[k][dd][j / 4][j % 4]); };
        // Every step issues one load per (tile, slot) in the same order, whether or
        // not the tile needs the block (an unneeded block's load reads nothing), so
        // the wait before each use stays a count of the loads issued after it.
#pragma unroll
        for (int dd = 0; dd < DEPTH; ++dd)
#pragma unroll
            for (int k = 0; k < TT; ++k) cb_load(k, 32 * dd, dd);
        // The loop runs DEPTH s blocks per iteration so that slot indices stay static,
        // up to the last block this wave's later live tile needs.
        const int kend = min(len, (live[1] ? t0_of[1] : t0_of[0]) + 16);
        for (int kb = 0; kb < kend; kb += 32 * DEPTH) {
#pragma unroll
            for (int dd = 0; dd < DEPTH; ++dd) {
                const int kk = kb + 32 * dd;
                if (kk >= kend) break;
                const int col = kk + kcol;
                v8 xf[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int pr = 16 * pt + lane % 16;
                    xf[pt] = *reinterpret_cast<const v8*>(xv + pr * XP + swz(pr, col));
                }
                // v_s exp2(ct - cs) = exp2(ct - (cs - log2 v_s)).
                float ls[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) ls[j] = sl[col + j];
#pragma unroll
                for (int k = 0; k < TT; ++k) {
                    const int t0 = t0_of[k];
                    if (live[k] && t0 + 15 >= kk) {
                        const int t = t0 + lane % 16;
                        const float ct = cum2[t];
                        v8 ah, al;  // the decayed entries' high and low parts
                        // Only the block that reaches the tile's rows needs the causal
                        // mask (s <= t); masked entries take exp2(-inf) = 0, a select.
                        // Rows past the chunk are computed from finite values and
                        // never stored.
                        if (kk + 31 > t0) {
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float ex = col + j <= t ? ct - ls[j] : -__builtin_huge_valf();
                                IT hi, lo;
                                split16(cb_value(k, dd, j) * __builtin_amdgcn_exp2f(ex), hi, lo);
                                ah[j] = hi;
                                al[j] = lo;
                            }
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                IT hi, lo;
                                split16(cb_value(k, dd, j) * __builtin_amdgcn_exp2f(ct - ls[j]), hi, lo);
                                ah[j] = hi;
                                al[j] = lo;
                            }
                        }
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) {
                            acc[k][pt] = Mfma<IT>::mma16(ah, xf[pt], acc[k][pt]);
                            acc[k][pt] = Mfma<IT>::mma16(al, xf[pt], acc[k][pt]);
                        }
                    }
                    cb_load(k, kk + 32 * DEPTH, dd);  // in flight during the next blocks
                }
            }
        }

        if (j + 1 < HL) issue(min(h + 1, H - 1));  // (a repeat of h past the last head is unused)
#pragma unroll
        for (int k = ZL; k < TT; ++k) z_load(k);

        // ---- skip term from the exact x^T in LDS (row t's four consecutive tokens
        // are one 8-byte read), then gate and store: each tile goes through a
        // wave-private LDS scratch spanning the entering-state and x^T areas (free
        // once every wave is past this point) so that z and out move as whole rows.
#pragma unroll
        for (int k = 0; k < TT; ++k)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                const int t = t0_of[k] + 4 * (lane / 16);
                typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
                const u16x4 xr4 = *reinterpret_cast<const u16x4*>(xv + pr * XP + swz(pr, t));
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[k][pt][i] += sd[pr] * f32_of<IT>(xr4[i]);
            }
        constexpr int EP = scan_epilogue_pitch(P);
        IT* op = static_cast<IT*>(p.out);
        const bool gate = p.z != nullptr;
        lds_barrier();  // every wave is done with x^T
        float* scratch = reinterpret_cast<float*>(xv) + wave * 16 * EP;
#pragma unroll
        for (int k = 0; k < TT; ++k) {
            if (!live[k]) break;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int i = 0; i < 4; ++i) scratch[(4 * (lane / 16) + i) * EP + 16 * pt + lane % 16] = acc[k][pt][i];
            ssu::wave_lds_sync();
            const u16x8 zz[2] = {k < ZL ? zslot[2 * 64 * NW * k] : ez[k][0],
                                 k < ZL ? zslot[2 * 64 * NW * k + 1] : ez[k][1]};
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int row = er + 8 * half, t = t0_of[k] + row;
                if (t < len) {
                    const f32x4* srow = reinterpret_cast<const f32x4*>(scratch + row * EP + ec);
                    u16x8 o;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float y = srow[e / 4][e % 4];
                        if (gate) y *= gate_f32(f32_of<IT>(zz[half][e]));
                        o[e] = bits_of<IT>(y);
                    }
                    __builtin_nontemporal_store(
                        o, reinterpret_cast<u16x8*>(op + xoff + static_cast<int64_t>(t) * H * PF + ec));
                }
            }
            ssu::wave_lds_sync();  // the next tile reuses the scratch
        }
    }  // heads
}

}  // namespace ssd

namespace ssd {

// The launches of one prefill, on `stream`: the front (request list, prep and
// C B^T), the state walk, the scan. Dispatches on the state type and the
// (headdim, dstate, chunk) instance.
template <typename IT, typename ST, int N, int Q>
hipError_t launch_instance(const SsdParams& p, hipStream_t stream) {
    constexpr int NB = N < kWalkStateBlock ? N : kWalkStateBlock;  // dstate block of a walk item
    const int64_t blocks = static_cast<int64_t>(p.headdim / kHeadBlock) * (N / NB);
    const int64_t front = front_blocks<Q>(p.nchunks, p.nheads, p.ngroups);
    if (front > 0x7fffffff || p.nchunks * p.nheads * (p.headdim / kHeadBlock) > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((ssd_front_kernel<IT, N, Q>), dim3(static_cast<unsigned>(front)),
                       dim3(kThreads), 0, stream, p);
    // The walk runs as many workgroups as fit on the device at once (each loops
    // over work items), never more than there can be items.
    // (Cached per device and instance; concurrent first calls store the same value.)
    static std::atomic<int> resident[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int fit = resident[dev].load(std::memory_order_relaxed);
    if (fit == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ssd_state_walk_kernel<IT, ST, NB, Q>,
                                                         walk_threads(NB), walk_lds_bytes(kHeadBlock, NB)) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidValue;
        fit = per_cu * cus > 0 ? per_cu * cus : 1;
        resident[dev].store(fit, std::memory_order_relaxed);
    }
    const int64_t walkers = std::min<int64_t>(fit, p.nchunks * p.nheads * blocks);
    hipLaunchKernelGGL((ssd_state_walk_kernel<IT, ST, NB, Q>), dim3(static_cast<unsigned>(walkers)),
                       dim3(walk_threads(NB)), walk_lds_bytes(kHeadBlock, NB), stream, p);
    constexpr int HL = scan_heads(N, Q);
    hipLaunchKernelGGL((ssd_scan_kernel<IT, ST, N, Q>),
                       dim3(static_cast<unsigned>(p.nchunks * ((p.nheads + HL - 1) / HL) *
                                                  (p.headdim / kHeadBlock))),
                       dim3(scan_threads(Q)), scan_lds_bytes(kHeadBlock, N, Q), stream, p);
    return hipGetLastError();
}

template <typename IT, typename ST>
hipError_t launch_shape(const SsdParams& p, int P, int N, int Q, hipStream_t stream) {
    if (P % kHeadBlock) return hipErrorInvalidValue;
    if (N == 128 && Q == 256) return launch_instance<IT, ST, 128, 256>(p, stream);
    if (N == 128 && Q == 128) return launch_instance<IT, ST, 128, 128>(p, stream);
    if (N == 64 && Q == 256) return launch_instance<IT, ST, 64, 256>(p, stream);
    if (N == 64 && Q == 128) return launch_instance<IT, ST, 64, 128>(p, stream);
    if (N == 256 && Q == 256) return launch_instance<IT, ST, 256, 256>(p, stream);
    if (N == 256 && Q == 128) return launch_instance<IT, ST, 256, 128>(p, stream);
    return hipErrorInvalidValue;
}

template <typename IT>
hipError_t launch_io(const SsdParams& p, int state_dtype, int P, int N, int Q, hipStream_t stream) {
    switch (state_dtype) {
        case kF32: return launch_shape<IT, float>(p, P, N, Q, stream);
        case kF16: return launch_shape<IT, _Float16>(p, P, N, Q, stream);
        case kBF16: return launch_shape<IT, __bf16>(p, P, N, Q, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ssd
