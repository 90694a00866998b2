// ssd_kernel.hpp -- SSD chunked prefill for gfx950 (CDNA4, wave64, MFMA).
//
// The prefill of a Mamba-2 layer over packed variable-length requests, cut into
// chunks of at most Q tokens (semantics in include/ssd.h), as five launches:
//
//   list      the requests whose last chunk is c, per chunk        (one workgroup)
//   bmm       CB[t, s] = C_t . B_s                                 per (chunk, group)
//   chunk     L_c = sum_s exp(cum_last - cum_s) v_s x_s B_s^T      per (chunk, head, block)
//   passing   S_c = exp(cum_last) S_{c-1} + L_c along each request per 4 state elements
//   scan      y_t = sum_{s<=t} CB[t, s] exp(cum_t - cum_s) v_s x_s
//                   + exp(cum_t) C_t . S_{c-1} + D x_t, gated      per (chunk, head)
//
// with v the clamped step and cum the running sum of A v inside the chunk
// (fp64, so the decay between two tokens is exact to fp32 however far into the
// chunk they lie). The three contractions run on the matrix cores with 16-bit
// operands and fp32 accumulation. The chunk kernel feeds exp(.) v x as a high
// and a low 16-bit part, which makes each product of a state accurate to about
// 2^-16 instead of 2^-8; the scan rounds its decayed C B^T entries once and uses
// x exactly. An opening chunk's L already carries the decayed initial state, so
// the passing walk is a chain of FMAs over loads requested chunks ahead. The
// passing kernel writes each chunk-end state in the io type (the scan's 16-bit
// MFMA operand) and in the state type where the caller asked for it.
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

#include "ssu_kernel.hpp"

namespace ssd {

using ssu::lds_barrier;
using ssu::load_index;
using ssu::silu_f32;
using ssu::softplus_f32;
using ssu::uniform64;

constexpr int kThreads = 256;  // four wave64s per workgroup
constexpr int kWaves = kThreads / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// dtype codes of include/ssu.h.
enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

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
    void* s16;            // workspace [nchunks, H, P, N] io: chunk-end states for the scan
    float* cb;            // workspace [nchunks, G, Q, Q]
    float* local;         // workspace [nchunks, H, P, N]: each chunk's own state contribution
    float* cumlast;       // workspace [nchunks, H]: each chunk's decay exponent
    void* dummy;          // workspace [H, P, N] state type: sink of steps with nothing to return
    int* list_head;       // workspace [nchunks]: first request whose last chunk is c
    int* list_next;       // workspace [batch]
    int64_t tokens, nchunks, batch;
    float dt_min, dt_max;
    int32_t nheads, ngroups, heads_per_group;
    int32_t dt_dtype;
    int32_t meta_i64;
    int32_t D_per_dim, dt_softplus;
    int32_t return_all;   // states[c] for every chunk instead of states[b] per request
    int32_t state_heads;  // heads per chunk-state workgroup: divides heads_per_group, <= 4
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

// Storage of the per-chunk C B^T entries: bf16 when the io type is bf16 (the
// scan rounds them to bf16 for the matrix cores anyway, after the decay), fp32
// for fp16 io, whose finer rounding a bf16 copy would spoil.
template <typename IT> struct CbStore { typedef float type; };
template <> struct CbStore<__bf16> { typedef __bf16 type; };

// 16-bit io value <-> bits <-> fp32.
template <typename T>
__device__ __forceinline__ float f32_of(unsigned short b) {
    return static_cast<float>(__builtin_bit_cast(T, b));
}
template <typename T>
__device__ __forceinline__ unsigned short bits_of(float v) {
    return __builtin_bit_cast(unsigned short, static_cast<T>(v));
}

// One state-type element <-> fp32.
template <typename ST>
__device__ __forceinline__ float load_state(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const ST*>(p)[i]);
}
template <typename ST>
__device__ __forceinline__ void store_state(void* p, int64_t i, float v) {
    static_cast<ST*>(p)[i] = static_cast<ST>(v);
}

__device__ __forceinline__ float load_dt(const SsdParams& p, int64_t i) {
    if (p.dt_dtype == kF32) return static_cast<const float*>(p.dt)[i];
    if (p.dt_dtype == kF16) return static_cast<float>(static_cast<const _Float16*>(p.dt)[i]);
    return static_cast<float>(static_cast<const __bf16*>(p.dt)[i]);
}

// Streaming data (x, z, out, the chunk contributions) is read and written
// non-temporally, so that it does not push the operands every head of a group
// shares (B, C, C B^T of the chunk) out of L2.
__device__ __forceinline__ u16x8 stream_load(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u16x8*>(p));
}

// Workgroups are dealt round robin to the XCDs, each with its own L2. Renumber
// them so that each XCD walks a contiguous range of chunk-major tiles: all heads
// of a chunk then meet the chunk's shared operands in one L2.
__device__ __forceinline__ int64_t xcd_order(int64_t id, int64_t n) { return ssu::xcd_tile(id, n); }

// Chunk c's first token and length; a range outside [0, tokens], running
// backwards or longer than Q counts as empty.
struct Chunk {
    int64_t lo;
    int len;
};

template <int Q>
__device__ __forceinline__ Chunk chunk_of(const SsdParams& p, int64_t c) {
    const int64_t lo = uniform64(load_index(p.cu_chunk, p.meta_i64, c));
    const int64_t hi = uniform64(load_index(p.cu_chunk, p.meta_i64, c + 1));
    if (lo < 0 || hi < lo || hi > p.tokens || hi - lo > Q) return {0, 0};
    return {lo, static_cast<int>(hi - lo)};
}

// The raw step of token `tid` of the chunk for head h (0 past the chunk): the
// load half of chunk_steps, so that it can be issued ahead of other loads.
__device__ __forceinline__ float load_step(const SsdParams& p, const Chunk& ch, int h) {
    const int tid = threadIdx.x;
    return tid < ch.len ? load_dt(p, (ch.lo + tid) * p.nheads + h) : 0.f;
}

// Per chunk and head: the clamped step v_s and the inclusive running sum
// cum_s = sum_{j<=s} A v_j (fp64) for s < len, into LDS; zero past len. `u` is
// this thread's load_step(). Every thread of the workgroup calls it; it ends
// with a barrier.
template <int Q, int THREADS = kThreads>
__device__ __forceinline__ void chunk_steps(const SsdParams& p, const Chunk& ch, int h, float u,
                                            float* sv, double* scum, double* swave) {
    static_assert(Q <= THREADS, "one step per thread");
    const int tid = threadIdx.x, lane = tid & 63;
    float v = 0.f;
    double a = 0.0;
    if (tid < ch.len) {
        if (p.dt_bias) u += p.dt_bias[h];
        if (p.dt_softplus) u = softplus_f32(u);
        u = fminf(fmaxf(u, p.dt_min), p.dt_max);
        v = u;
        a = static_cast<double>(p.A[h]) * static_cast<double>(u);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(a, d);
        if (lane >= d) a += o;
    }
    if (lane == 63) swave[tid >> 6] = a;
    lds_barrier();
    double off = 0.0;
    for (int w = 0; w < (tid >> 6); ++w) off += swave[w];
    if (tid < Q) {
        sv[tid] = v;
        scum[tid] = a + off;
    }
    lds_barrier();
}

// ------------------------------------------------------------ request list

// list_head[c] / list_next[b]: the requests b whose last chunk index is c, as a
// linked list per chunk (order unspecified; each b appears once). One workgroup.
template <int kUnused = 0>
__global__ __launch_bounds__(1024) void ssd_list_kernel(const SsdParams p) {
    for (int64_t c = threadIdx.x; c < p.nchunks; c += 1024) p.list_head[c] = -1;
    __syncthreads();
    for (int64_t b = threadIdx.x; b < p.batch; b += 1024) {
        const int64_t c = load_index(p.lci, p.meta_i64, b);
        if (c >= 0 && c < p.nchunks) p.list_next[b] = atomicExch(&p.list_head[c], static_cast<int>(b));
    }
}

// --------------------------------------------------------------------- bmm

// CB[c, g] = C B^T over the chunk's tokens, lower triangle of 32x32 tiles
// (s <= t needs no more), 32x32x16 MFMA with both operands straight from HBM
// (eight consecutive dstate values per lane are contiguous). Rows past the
// chunk's length read its last token and are never used.
template <typename IT, int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_bmm_kernel(const SsdParams p) {
    typedef typename Mfma<IT>::v8 v8;
    constexpr int TQ = Q / 32;
    const int64_t c = blockIdx.x / p.ngroups;
    const int g = blockIdx.x % p.ngroups;
    const Chunk ch = chunk_of<Q>(p, c);
    if (ch.len == 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const IT* Cp = static_cast<const IT*>(p.C);
    const IT* Bp = static_cast<const IT*>(p.B);
    typedef typename CbStore<IT>::type CBT;
    CBT* out = reinterpret_cast<CBT*>(p.cb) + (c * p.ngroups + g) * Q * Q;
    int tile = 0;
    for (int ti = 0; ti < TQ; ++ti) {
        for (int sj = 0; sj <= ti; ++sj, ++tile) {
            if (tile % kWaves != wave || ti * 32 >= ch.len) continue;
            const int t = min(ti * 32 + lane % 32, ch.len - 1);
            const int s = min(sj * 32 + lane % 32, ch.len - 1);
            const v8* ca = reinterpret_cast<const v8*>(Cp + ((ch.lo + t) * p.ngroups + g) * N);
            const v8* bb = reinterpret_cast<const v8*>(Bp + ((ch.lo + s) * p.ngroups + g) * N);
            f32x16 acc = {};
#pragma unroll
            for (int k = 0; k < N / 16; ++k)
                acc = Mfma<IT>::mma32(ca[2 * k + lane / 32], bb[2 * k + lane / 32], acc);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = ti * 32 + 8 * (i / 4) + 4 * (lane / 32) + i % 4;
                out[row * Q + sj * 32 + lane % 32] = static_cast<CBT>(acc[i]);
            }
        }
    }
}

// ------------------------------------------------------------------- state

// Transposed tiles in LDS keep the 16-byte chunks of each row permuted by the
// row's octet: chunk c of row r lives at chunk c ^ ((r / 8) % 8). The
// transposing stores (eight rows at once) then spread over the banks, and a
// fragment read (eight consecutive values of one row) stays one 16-byte access.
// Rows hold a multiple of 64 elements, so the permutation stays inside the row.
__device__ __forceinline__ int swz(int r, int col) {
    return (((col >> 3) ^ ((r >> 3) & 7)) << 3) | (col & 7);
}

// The chunk-state kernel: one workgroup per (chunk, block of `state_heads`
// heads of one group, half of the headdim rows) computes each head's own
// contribution to the state, L_c = sum_s exp(cum_last - cum_s) v_s x_s B_s^T
// (fp32, into the workspace), and (first half) the chunk's decay exponent per
// head. The heads share the chunk's B, staged once per block of KB tokens, and
// run as a pipeline: the steps of every head are requested together, and the
// next head's x is in flight while the current head's products run. It runs
// N / 16 waves; wave w owns dstate column tile w for the half's rows.
constexpr int kStateKB = 128;
constexpr int kStateRows = 32;             // headdim rows per workgroup
constexpr int kStateHeads = 4;             // most heads per workgroup
constexpr int kStatePitch = kStateKB + 8;  // LDS row pitch of the transposed tiles
__host__ __device__ constexpr int state_threads(int N) { return 4 * N; }

// LDS bytes of the chunk-state kernel: sv, scum, swave (the step scan of one
// head), the weights of every head, x^T high and low parts [rows][pitch] of one
// head and B^T [N][pitch]; the x^T area later holds one head's fp32 output tile.
__host__ __device__ constexpr unsigned state_lds_bytes(int N, int Q) {
    return 4u * Q + 8u * Q + 8u * (state_threads(N) / 64) + 4u * kStateHeads * Q +
           2u * (2 * kStateRows + N) * kStatePitch;
}

template <typename IT, typename ST, int P, int N, int Q>
__global__ __launch_bounds__(state_threads(N)) void ssd_chunk_state_kernel(const SsdParams p) {
    typedef typename Mfma<IT>::v8 v8;
    constexpr int NT = state_threads(N), NW = NT / 64;
    constexpr int PS = kStateRows, NS = N, KB = kStateKB, XP = kStatePitch, HM = kStateHeads;
    constexpr int PB = P / PS;                        // row halves
    constexpr int PT = PS / 16;                       // row tiles
    static_assert(NS / 16 == NW && P % PS == 0, "one column tile per wave");
    constexpr int XQ = PS / 8, BQ = NS / 8;           // 16-byte pieces of a token's x / B row
    constexpr int XN = (KB / 2) * XQ, BN = (KB / 2) * BQ;  // two-token loads per block
    constexpr int XPASS = (XN + NT - 1) / NT, BPASS = (BN + NT - 1) / NT;
    constexpr int NSB = Q / KB > 0 ? Q / KB : 1;      // token blocks per chunk
    constexpr int OP = NS + 4;                        // output tile row pitch (floats)
    static_assert(PS * OP * 4 <= 2 * 2 * PS * XP, "output tile fits the x^T area");
    static_assert(Q <= NT, "one step per thread");

    const int HB = p.state_heads;
    int64_t wg = xcd_order(blockIdx.x, gridDim.x);
    const int pb = static_cast<int>(wg % PB);
    wg /= PB;
    const int hblocks = p.nheads / HB;
    const int h0 = static_cast<int>(wg % hblocks) * HB;
    const int64_t c = wg / hblocks;
    const int g = h0 / p.heads_per_group;
    const int H = p.nheads;
    const int p0 = pb * PS;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sv = reinterpret_cast<float*>(smem);
    double* scum = reinterpret_cast<double*>(sv + Q);
    double* swave = scum + Q;
    float* sw = reinterpret_cast<float*>(swave + NW);   // [HM][Q]
    unsigned short* xhi = reinterpret_cast<unsigned short*>(sw + HM * Q);
    unsigned short* xlo = xhi + PS * XP;
    unsigned short* bt = xlo + PS * XP;
    float* oblk = reinterpret_cast<float*>(xhi);

    const IT* xp = static_cast<const IT*>(p.x);
    const IT* Bp = static_cast<const IT*>(p.B);
    const Chunk ch = chunk_of<Q>(p, c);

    // Staged registers: x of one (head, block), B of one block.
    u16x8 rx[XPASS][2], rb[BPASS][2];
    auto fetch_x = [&](int hh, int sb) {
        const int s0 = KB * sb, h = h0 + hh;
#pragma unroll
        for (int r = 0; r < XPASS; ++r) {
            const int idx = tid + NT * r, q = idx % XQ, s = s0 + 2 * (idx / XQ);
            const bool on = idx < XN;
            const IT* row = xp + ((ch.lo + s) * H + h) * P + p0 + 8 * q;
            rx[r][0] = on && s < ch.len ? stream_load(row) : u16x8{};
            rx[r][1] = on && s + 1 < ch.len ? stream_load(row + H * P) : u16x8{};
        }
    };
    auto fetch_b = [&](int sb) {
        const int s0 = KB * sb;
#pragma unroll
        for (int r = 0; r < BPASS; ++r) {
            const int idx = tid + NT * r, q = idx % BQ, s = s0 + 2 * (idx / BQ);
            const bool on = idx < BN;
            const IT* row = Bp + ((ch.lo + s) * p.ngroups + g) * N + 8 * q;
            rb[r][0] = on && s < ch.len ? *reinterpret_cast<const u16x8*>(row) : u16x8{};
            rb[r][1] = on && s + 1 < ch.len ? *reinterpret_cast<const u16x8*>(row + p.ngroups * N) : u16x8{};
        }
    };

    // The steps of every head first, then the first blocks of B and x.
    float u[HM];
#pragma unroll
    for (int hh = 0; hh < HM; ++hh) u[hh] = hh < HB ? load_step(p, ch, h0 + hh) : 0.f;
    fetch_b(0);
    fetch_x(0, 0);

    float decay[HM];
#pragma unroll
    for (int hh = 0; hh < HM; ++hh) {
        if (hh >= HB) break;
        lds_barrier();  // the previous head's scan is consumed
        chunk_steps<Q, NT>(p, ch, h0 + hh, u[hh], sv, scum, swave);
        const double last = ch.len > 0 ? scum[ch.len - 1] : 0.0;
        if (tid < Q)
            sw[hh * Q + tid] = tid < ch.len ? expf(static_cast<float>(last - scum[tid])) * sv[tid] : 0.f;
        if (pb == 0 && tid == 0) p.cumlast[c * H + h0 + hh] = static_cast<float>(last);
        decay[hh] = expf(static_cast<float>(last));
    }

    f32x4 acc[HM][PT];
#pragma unroll
    for (int hh = 0; hh < HM; ++hh)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[hh][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        const int s0 = KB * sb;
        if (s0 >= ch.len) break;
        lds_barrier();  // the previous block's B^T is consumed; sw visible
#pragma unroll
        for (int r = 0; r < BPASS; ++r) {
            const int idx = tid + NT * r, q = idx % BQ, j = 2 * (idx / BQ);
            if (idx >= BN) break;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 8 * q + e;
                *reinterpret_cast<unsigned*>(bt + row * XP + swz(row, j)) =
                    rb[r][0][e] | (static_cast<unsigned>(rb[r][1][e]) << 16);
            }
        }
        if (sb + 1 < NSB && s0 + KB < ch.len) fetch_b(sb + 1);
#pragma unroll
        for (int hh = 0; hh < HM; ++hh) {
            if (hh >= HB) break;
            if (hh > 0) lds_barrier();  // the previous head's products are done with x^T
            // x^T of head hh (scaled by its weights, high and low parts) into LDS.
            const float* swh = sw + hh * Q + s0;
#pragma unroll
            for (int r = 0; r < XPASS; ++r) {
                const int idx = tid + NT * r, q = idx % XQ, j = 2 * (idx / XQ);
                if (idx >= XN) break;
                const float w0 = s0 + j < ch.len ? swh[j] : 0.f;
                const float w1 = s0 + j + 1 < ch.len ? swh[j + 1] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a0 = f32_of<IT>(rx[r][0][e]) * w0;
                    const float a1 = f32_of<IT>(rx[r][1][e]) * w1;
                    const unsigned short hi0 = bits_of<IT>(a0), hi1 = bits_of<IT>(a1);
                    const unsigned short lo0 = bits_of<IT>(a0 - f32_of<IT>(hi0));
                    const unsigned short lo1 = bits_of<IT>(a1 - f32_of<IT>(hi1));
                    const int row = 8 * q + e, o = row * XP + swz(row, j);
                    *reinterpret_cast<unsigned*>(xhi + o) = hi0 | (static_cast<unsigned>(hi1) << 16);
                    *reinterpret_cast<unsigned*>(xlo + o) = lo0 | (static_cast<unsigned>(lo1) << 16);
                }
            }
            // The next head's x (or the next block's first head) is requested now.
            if (hh + 1 < HB)
                fetch_x(hh + 1, sb);
            else if (sb + 1 < NSB && s0 + KB < ch.len)
                fetch_x(0, sb + 1);
            lds_barrier();
#pragma unroll
            for (int kk = 0; kk < KB; kk += 32) {
                if (s0 + kk >= ch.len) break;
                const int col = kk + 8 * (lane / 16);
                const int brow = 16 * wave + lane % 16;
                const v8 bf = *reinterpret_cast<const v8*>(bt + brow * XP + swz(brow, col));
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int row = 16 * pt + lane % 16, o = row * XP + swz(row, col);
                    acc[hh][pt] = Mfma<IT>::mma16(*reinterpret_cast<const v8*>(xhi + o), bf, acc[hh][pt]);
                    acc[hh][pt] = Mfma<IT>::mma16(*reinterpret_cast<const v8*>(xlo + o), bf, acc[hh][pt]);
                }
            }
        }
    }

    // Each head's L_c through LDS, so that each wave store covers whole rows. A
    // chunk that opens a request with an initial state h0 stores
    // exp(cum_last) h0 + L_c instead: the state after it.
    const int64_t req = uniform64(load_index(p.seq_idx, p.meta_i64, c));
    const bool opens = c == 0 || req != load_index(p.seq_idx, p.meta_i64, c - 1);
    const bool fold = opens && p.init && req >= 0 && req < p.batch;
    constexpr int OPASS = PS * NS / 4 / NT;  // four-float pieces per thread
    static_assert(OPASS * NT * 4 == PS * NS, "output passes");
#pragma unroll
    for (int hh = 0; hh < HM; ++hh) {
        if (hh >= HB) break;
        const int h = h0 + hh;
        lds_barrier();  // x^T (or the previous head's tile) is consumed
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oblk[(16 * pt + 4 * (lane / 16) + i) * OP + 16 * wave + lane % 16] = acc[hh][pt][i];
        lds_barrier();
        float* const dst_tile = p.local + ((c * H + h) * P + p0) * static_cast<int64_t>(NS);
#pragma unroll
        for (int r = 0; r < OPASS; ++r) {
            const int idx = 4 * (tid + NT * r), orow = idx / NS, ocol = idx % NS;
            f32x4 v = *reinterpret_cast<const f32x4*>(oblk + orow * OP + ocol);
            if (fold) {
                const int64_t base = ((req * H + h) * P + p0 + orow) * static_cast<int64_t>(N) + ocol;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = fmaf(decay[hh], load_state<ST>(p.init, base + j), v[j]);
            }
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst_tile + idx));
        }
    }
}

// State passing: thread owns four consecutive elements of one head's state and
// walks all chunks in order: a chunk that opens a request takes its stored
// value as the state (it already holds the initial state's decayed
// contribution), every other chunk applies S = exp(cum_last) S + L_c. The chunk
// values are requested kPassDepth chunks ahead and every step makes the same
// memory accesses (one load, two stores; a step with nothing to return writes
// its state to a private dummy slot), so the loads stay in flight across steps.
// S leaves in the io type for the scan of the next chunk, and in the state type
// for chunk c (every chunk) or for the first request whose last chunk is c;
// ssd_fixup_kernel copies it to further requests naming the same chunk.
constexpr int kPassThreads = 256;
constexpr int kPassDepth = 8;

template <typename IT, typename ST, int P, int N>
__global__ __launch_bounds__(kPassThreads) void ssd_state_passing_kernel(const SsdParams p) {
    constexpr int PER_HEAD = P * N / 4;  // threads per head
    static_assert(PER_HEAD % kPassThreads == 0, "a workgroup stays in one head");
    constexpr int W = kPassThreads;      // chunks whose metadata one LDS window holds
    static_assert(W % kPassDepth == 0, "windows hold whole blocks");
    typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
    typedef ST st4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int64_t gt = static_cast<int64_t>(blockIdx.x) * kPassThreads + tid;
    const int h = __builtin_amdgcn_readfirstlane(static_cast<int>(gt / PER_HEAD));
    const int64_t e = (gt % PER_HEAD) * 4;        // element within the head's state
    const int H = p.nheads;
    const int64_t tile = static_cast<int64_t>(H) * P * N;
    const int64_t he = static_cast<int64_t>(h) * P * N + e;
    ST* const dummy = static_cast<ST*>(p.dummy) + he;
    const int64_t last = p.nchunks - 1;

    // Metadata of a window of W chunks, staged in LDS (LDS reads do not wait on
    // the vector-memory counter the prefetched loads are tracked by): whether the
    // chunk opens a request, its decay, and where its state is returned (-1: not).
    __shared__ int s_open[W];
    __shared__ float s_decay[W];
    __shared__ int64_t s_dest[W];

    f32x4 ring[kPassDepth];
#pragma unroll
    for (int j = 0; j < kPassDepth; ++j)
        ring[j] = *reinterpret_cast<const f32x4*>(p.local + min<int64_t>(j, last) * tile + he);
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    for (int64_t w0 = 0; w0 < p.nchunks; w0 += W) {
        __syncthreads();  // the previous window's metadata is consumed
        {
            const int64_t c = w0 + tid;
            if (c <= last) {
                const int64_t r = load_index(p.seq_idx, p.meta_i64, c);
                s_open[tid] = c == 0 || r != load_index(p.seq_idx, p.meta_i64, c - 1);
                s_decay[tid] = expf(p.cumlast[c * H + h]);
                const int64_t b = p.return_all ? c : p.list_head[c];
                s_dest[tid] = (b >= 0 && b < (p.return_all ? p.nchunks : p.batch)) ? b : -1;
            }
        }
        __syncthreads();
        // Branch-free steps (selects and clamped or dummy addresses), so the
        // compiler can keep the ring's loads in flight across them.
        for (int64_t c0 = w0; c0 < w0 + W && c0 <= last; c0 += kPassDepth) {
#pragma unroll
            for (int j = 0; j < kPassDepth; ++j) {
                const int64_t c = c0 + j;
                const bool valid = c <= last;
                const int k = valid ? static_cast<int>(c - w0) : 0;
                const f32x4 local = ring[j];
                ring[j] = *reinterpret_cast<const f32x4*>(
                    p.local + min<int64_t>(c + kPassDepth, last) * tile + he);
                const bool open = s_open[k] != 0;
                const float d = s_decay[k];
#pragma unroll
                for (int i = 0; i < 4; ++i) S[i] = open ? local[i] : fmaf(d, S[i], local[i]);
                u16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = bits_of<IT>(S[i]);
                IT* s16 = valid ? static_cast<IT*>(p.s16) + c * tile + he
                                : reinterpret_cast<IT*>(dummy);
                *reinterpret_cast<u16x4*>(s16) = o;
                const int64_t b = valid ? s_dest[k] : -1;
                ST* dst = b >= 0 ? static_cast<ST*>(p.states) + b * tile + he : dummy;
                st4 q;
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = static_cast<ST>(S[i]);
                *reinterpret_cast<st4*>(dst) = q;
            }
        }
    }
}

// Requests whose last chunk is also another request's (only an inconsistent
// caller makes two requests name one chunk) get that request's returned state.
// One workgroup per request.
template <typename ST, int P, int N>
__global__ __launch_bounds__(kPassThreads) void ssd_fixup_kernel(const SsdParams p) {
    const int64_t b = blockIdx.x;
    const int64_t c = load_index(p.lci, p.meta_i64, b);
    if (c < 0 || c >= p.nchunks) return;
    const int64_t first = p.list_head[c];
    if (first == b || first < 0 || first >= p.batch) return;
    const int64_t tile = static_cast<int64_t>(p.nheads) * P * N;
    const ST* src = static_cast<const ST*>(p.states) + first * tile;
    ST* dst = static_cast<ST*>(p.states) + b * tile;
    for (int64_t i = threadIdx.x; i < tile; i += kPassThreads) dst[i] = src[i];
}

// -------------------------------------------------------------------- scan

// The scan runs Q / 32 waves: two 16-token tiles of the chunk per wave.
__host__ __device__ constexpr int scan_threads(int Q) { return 2 * Q; }
constexpr int scan_pitch(int Q) { return Q + 8; }       // (v x)^T row pitch, elements
constexpr int state_pitch(int N) { return N + 8; }      // entering-state row pitch

// LDS bytes of the scan kernel: sv, the log2-scaled running sums (fp32), the
// fp64 running sums, one fp64 per wave, the entering state [P][N + 8] and
// (v x)^T [P][Q + 8], both in the io type.
__host__ __device__ constexpr unsigned scan_lds_bytes(int P, int N, int Q) {
    return 4u * Q + 4u * Q + 8u * Q + 8u * (scan_threads(Q) / 64) + 2u * P * state_pitch(N) +
           2u * P * scan_pitch(Q);
}

// (v x)^T and the entering state are stored permuted by swz().

// One workgroup per (chunk, head); wave w owns token tiles w and w + Q / 32.
// Independent loads are issued before anything waits: the x tile, the entering
// state and the first C operands at the start, each product's next operands
// before its current matrix-core work.
template <typename IT, typename ST, int P, int N, int Q>
__global__ __launch_bounds__(scan_threads(Q)) void ssd_scan_kernel(const SsdParams p) {
    typedef typename Mfma<IT>::v8 v8;
    constexpr int NT = scan_threads(Q), NW = NT / 64;
    constexpr int PT = P / 16, TT = 2, KN = N / 32;
    constexpr int XP = scan_pitch(Q), SP = state_pitch(N);
    constexpr int XPASS = (Q / 2) * (P / 8) / NT;   // x loads per thread (token pairs x row octets)
    constexpr int SPASS = P * (N / 8) / NT;         // entering-state 16-byte chunks per thread
    static_assert(XPASS * NT == (Q / 2) * (P / 8) && SPASS * NT == P * (N / 8), "passes");
    static_assert((SP * 2) % 16 == 0 && (XP * 2) % 16 == 0, "16-byte rows");
    constexpr float kLog2e = 1.4426950408889634f;

    const int64_t wg = xcd_order(blockIdx.x, gridDim.x);
    const int64_t c = wg / p.nheads;
    const int h = static_cast<int>(wg % p.nheads);
    const Chunk ch = chunk_of<Q>(p, c);
    if (ch.len == 0) return;
    const int g = h / p.heads_per_group;
    const int H = p.nheads;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sv = reinterpret_cast<float*>(smem);
    float* cum2 = sv + Q;
    double* scum = reinterpret_cast<double*>(cum2 + Q);
    double* swave = scum + Q;
    unsigned short* sS = reinterpret_cast<unsigned short*>(swave + NW);
    unsigned short* xv = sS + P * SP;

    const IT* xp = static_cast<const IT*>(p.x);
    const IT* Cp = static_cast<const IT*>(p.C);

    // ---- loads issued up front: the steps, the x tile, the entering state and
    // the first C operands.
    const float u = load_step(p, ch, h);
    // x: thread handles row octet q of token pair jp (eight threads per token row).
    u16x8 rx[XPASS][2];
#pragma unroll
    for (int r = 0; r < XPASS; ++r) {
        const int idx = tid + NT * r, q = idx % (P / 8), s = 2 * (idx / (P / 8));
        const IT* row = xp + ((ch.lo + s) * H + h) * P + 8 * q;
        rx[r][0] = s < ch.len ? stream_load(row) : u16x8{};
        rx[r][1] = s + 1 < ch.len ? stream_load(row + H * P) : u16x8{};
    }
    // The entering state: the previous chunk's (io type) or the request's initial state.
    const int64_t req = uniform64(load_index(p.seq_idx, p.meta_i64, c));
    const bool opens = c == 0 || req != load_index(p.seq_idx, p.meta_i64, c - 1);
    const bool from_init = opens && p.init && req >= 0 && req < p.batch;
    const bool has_state = !opens || from_init;
    u16x8 rs[SPASS];
#pragma unroll
    for (int r = 0; r < SPASS; ++r) {
        const int ci = tid + NT * r, pr = ci / (N / 8), n8 = 8 * (ci % (N / 8));
        if (!opens) {
            rs[r] = *reinterpret_cast<const u16x8*>(static_cast<const IT*>(p.s16) +
                                                    (((c - 1) * H + h) * P + pr) * N + n8);
        } else if (from_init) {
            const int64_t base = ((req * H + h) * P + pr) * N + n8;
#pragma unroll
            for (int j = 0; j < 8; ++j) rs[r][j] = bits_of<IT>(load_state<ST>(p.init, base + j));
        } else {
            rs[r] = u16x8{};
        }
    }
    // C operands of the entering-state product, first k step.
    int trow[TT];
#pragma unroll
    for (int k = 0; k < TT; ++k) trow[k] = min(16 * (wave + NW * k) + lane % 16, ch.len - 1);
    const int kcol = 8 * (lane / 16);
    auto c_frag = [&](int k, int kk) {
        return *reinterpret_cast<const v8*>(Cp + ((ch.lo + trow[k]) * p.ngroups + g) * N + kk + kcol);
    };
    v8 cf[TT];
    if (has_state) {
#pragma unroll
        for (int k = 0; k < TT; ++k) cf[k] = c_frag(k, 0);
    }

    chunk_steps<Q, NT>(p, ch, h, u, sv, scum, swave);
    if (tid < Q) cum2[tid] = static_cast<float>(scum[tid]) * kLog2e;

    // x^T (exact) and the entering state into LDS.
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
        *reinterpret_cast<u16x8*>(sS + pr * SP + swz(pr, n8)) = rs[r];
    }
    lds_barrier();

    f32x4 acc[TT][PT];
#pragma unroll
    for (int k = 0; k < TT; ++k)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool live[TT];
#pragma unroll
    for (int k = 0; k < TT; ++k) live[k] = 16 * (wave + NW * k) < ch.len;

    // ---- the entering state: C_t . S_in, then scaled by exp(cum_t)
    if (has_state) {
#pragma unroll
        for (int ks = 0; ks < KN; ++ks) {
            v8 cn[TT];
            if (ks + 1 < KN) {
#pragma unroll
                for (int k = 0; k < TT; ++k) cn[k] = c_frag(k, 32 * (ks + 1));
            }
            v8 sf[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                sf[pt] = *reinterpret_cast<const v8*>(sS + pr * SP + swz(pr, 32 * ks + kcol));
            }
#pragma unroll
            for (int k = 0; k < TT; ++k)
                if (live[k])
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[k][pt] = Mfma<IT>::mma16(cf[k], sf[pt], acc[k][pt]);
            if (ks + 1 < KN) {
#pragma unroll
                for (int k = 0; k < TT; ++k) cf[k] = cn[k];
            }
        }
#pragma unroll
        for (int k = 0; k < TT; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = min(16 * (wave + NW * k) + 4 * (lane / 16) + i, Q - 1);
                const float f = __builtin_amdgcn_exp2f(cum2[t]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[k][pt][i] *= f;
            }
    }

    // ---- inside the chunk: (C B^T masked, times the decays and the steps v_s)
    // times x. Tile k needs the s blocks kk <= its last row; its C B^T entries
    // are requested two blocks ahead of their products.
    typedef typename CbStore<IT>::type CBT;
    const CBT* cbp = reinterpret_cast<const CBT*>(p.cb) + (c * p.ngroups + g) * Q * Q;
    // Eight C B^T entries of one row: one 16-byte load for bf16, two for fp32.
    constexpr int CW = sizeof(CBT) == 2 ? 1 : 2;
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    constexpr int DEPTH = 2;  // s blocks of C B^T in flight per tile
    u32x4v cb[TT][DEPTH][CW];
    // Tile k's C B^T entries of s block kk into slot d, if the tile needs that block.
    auto cb_load = [&](int k, int kk, int d) {
        const int t0 = 16 * (wave + NW * k);
        if (live[k] && t0 + 15 >= kk && kk < ch.len) {
            const u32x4v* r =
                reinterpret_cast<const u32x4v*>(cbp + (t0 + lane % 16) * Q + kk + kcol);
#pragma unroll
            for (int w = 0; w < CW; ++w) cb[k][d][w] = r[w];
        }
    };
    auto cb_value = [&](int k, int d, int j) -> float {
        if constexpr (CW == 1) {
            const unsigned word = cb[k][d][0][j / 2];
            return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
        } else {
            return __uint_as_float(cb[k][d][j / 4][j % 4]);
        }
    };
#pragma unroll
    for (int k = 0; k < TT; ++k)
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) cb_load(k, 32 * d, d);
    // The loop runs DEPTH s blocks per iteration so that slot indices stay static.
    for (int kb = 0; kb < ch.len; kb += 32 * DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int kk = kb + 32 * d;
            if (kk >= ch.len) break;
            const int col = kk + kcol;
            v8 xf[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                xf[pt] = *reinterpret_cast<const v8*>(xv + pr * XP + swz(pr, col));
            }
            float cs[8], vs[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                cs[j] = cum2[col + j];
                vs[j] = sv[col + j];
            }
#pragma unroll
            for (int k = 0; k < TT; ++k) {
                const int t0 = 16 * (wave + NW * k);
                if (!live[k] || t0 + 15 < kk) continue;
                const int t = t0 + lane % 16;
                const float ct = cum2[t];
                v8 a;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float m = cb_value(k, d, j);
                    const bool on = col + j <= t && t < ch.len;
                    a[j] = static_cast<IT>(on ? m * vs[j] * __builtin_amdgcn_exp2f(ct - cs[j]) : 0.f);
                }
                cb_load(k, kk + 32 * DEPTH, d);  // in flight during the next blocks
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[k][pt] = Mfma<IT>::mma16(a, xf[pt], acc[k][pt]);
            }
        }
    }

    // z rows of the epilogue, requested before the skip term: lane l finishes 16
    // consecutive columns of row l / 4 of each of its tiles.
    const IT* zp = static_cast<const IT*>(p.z);
    const int er = lane / 4, ec = (lane % 4) * (P / 4);
    static_assert(P / 4 == 16, "one lane finishes 16 columns");
    u16x8 ez[TT][2];
    if (zp) {
#pragma unroll
        for (int k = 0; k < TT; ++k) {
            const int t = min(16 * (wave + NW * k) + er, ch.len - 1);
            const IT* zr = zp + ((ch.lo + t) * H + h) * P + ec;
            ez[k][0] = stream_load(zr);
            ez[k][1] = stream_load(zr + 8);
        }
    }
    // ---- skip term from the exact x^T in LDS (row t's four consecutive tokens
    // are one 8-byte read), then gate and store: each tile goes through a
    // wave-private LDS scratch spanning the entering-state and x^T areas (free
    // once every wave is past this point) so that z and out move as whole rows.
    if (p.D) {
#pragma unroll
        for (int k = 0; k < TT; ++k)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                const int t = 16 * (wave + NW * k) + 4 * (lane / 16);
                typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
                const u16x4 xr = *reinterpret_cast<const u16x4*>(xv + pr * XP + swz(pr, t));
                const float d = p.D_per_dim ? p.D[h * P + pr] : p.D[h];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[k][pt][i] += d * f32_of<IT>(xr[i]);
            }
    }
    constexpr int EP = P + 4;  // scratch row pitch in floats (16-byte aligned rows)
    static_assert(NW * 16 * EP * 4 <= 2 * P * (SP + XP), "epilogue scratch fits");
    IT* op = static_cast<IT*>(p.out);
    lds_barrier();
    float* scratch = reinterpret_cast<float*>(sS) + wave * 16 * EP;
#pragma unroll
    for (int k = 0; k < TT; ++k) {
        if (!live[k]) break;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) scratch[(4 * (lane / 16) + i) * EP + 16 * pt + lane % 16] = acc[k][pt][i];
        ssu::wave_lds_sync();
        const int t = 16 * (wave + NW * k) + er;
        if (t < ch.len) {
            const int64_t xi = ((ch.lo + t) * H + h) * P + ec;
            const f32x4* srow = reinterpret_cast<const f32x4*>(scratch + er * EP + ec);
            u16x8 o0, o1;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float y = srow[e / 4][e % 4];
                if (zp) y *= silu_f32(f32_of<IT>(ez[k][e / 8][e % 8]));
                if (e < 8)
                    o0[e] = bits_of<IT>(y);
                else
                    o1[e - 8] = bits_of<IT>(y);
            }
            __builtin_nontemporal_store(o0, reinterpret_cast<u16x8*>(op + xi));
            __builtin_nontemporal_store(o1, reinterpret_cast<u16x8*>(op + xi + 8));
        }
        ssu::wave_lds_sync();  // the next tile reuses the scratch
    }
}

}  // namespace ssd

namespace ssd {

// The four launches of one prefill, on `stream`: the request list (when final
// states are gathered per request), bmm, state, scan. Dispatches on the state
// type and the (headdim, dstate, chunk) instance.
template <typename IT, typename ST, int P, int N, int Q>
hipError_t launch_instance(const SsdParams& p, hipStream_t stream) {
    if (!p.return_all && p.batch > 0)
        hipLaunchKernelGGL(ssd_list_kernel<0>, dim3(1), dim3(1024), 0, stream, p);
    hipLaunchKernelGGL((ssd_bmm_kernel<IT, N, Q>), dim3(static_cast<unsigned>(p.nchunks * p.ngroups)),
                       dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((ssd_chunk_state_kernel<IT, ST, P, N, Q>),
                       dim3(static_cast<unsigned>(p.nchunks * (p.nheads / p.state_heads) *
                                                  (P / kStateRows))),
                       dim3(state_threads(N)), state_lds_bytes(N, Q), stream, p);
    hipLaunchKernelGGL((ssd_state_passing_kernel<IT, ST, P, N>),
                       dim3(static_cast<unsigned>(p.nheads * P * N / 4 / kPassThreads)),
                       dim3(kPassThreads), 0, stream, p);
    if (!p.return_all && p.batch > 0)
        hipLaunchKernelGGL((ssd_fixup_kernel<ST, P, N>), dim3(static_cast<unsigned>(p.batch)),
                           dim3(kPassThreads), 0, stream, p);
    hipLaunchKernelGGL((ssd_scan_kernel<IT, ST, P, N, Q>),
                       dim3(static_cast<unsigned>(p.nchunks * p.nheads)), dim3(scan_threads(Q)),
                       scan_lds_bytes(P, N, Q), stream, p);
    return hipGetLastError();
}

template <typename IT, typename ST>
hipError_t launch_shape(const SsdParams& p, int P, int N, int Q, hipStream_t stream) {
    if (P != 64) return hipErrorInvalidValue;
    if (N == 128 && Q == 256) return launch_instance<IT, ST, 64, 128, 256>(p, stream);
    if (N == 128 && Q == 128) return launch_instance<IT, ST, 64, 128, 128>(p, stream);
    if (N == 64 && Q == 256) return launch_instance<IT, ST, 64, 64, 256>(p, stream);
    if (N == 64 && Q == 128) return launch_instance<IT, ST, 64, 64, 128>(p, stream);
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
