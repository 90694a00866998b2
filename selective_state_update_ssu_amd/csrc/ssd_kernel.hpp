// ssd_kernel.hpp -- SSD chunked prefill for gfx950 (CDNA4, wave64, MFMA).
//
// The prefill of a Mamba-2 layer over packed variable-length requests, cut into
// chunks of at most Q tokens (semantics in include/ssd.h). Three contractions
// per chunk run on the matrix cores, with 16-bit operands and fp32 accumulation:
//
//   bmm    CB[t, s]  = C_t . B_s                         per (chunk, group)
//   state  S_c       = exp(cum_last) S_{c-1} + sum_s exp(cum_last - cum_s) v_s x_s B_s^T
//                                                         per (run of chunks, head)
//   scan   y_t       = sum_{s<=t} CB[t, s] exp(cum_t - cum_s) v_s x_s
//                      + exp(cum_t) C_t . S_{c-1} + D x_t, gated by z sigmoid(z)
//                                                         per (chunk, head)
//
// with v the clamped step and cum the running sum of A v inside the chunk. The
// state kernel walks each request's chunks in order, carrying the state in MFMA
// accumulators, so chunk states never make a round trip through HBM before they
// are passed on; it writes each chunk-end state once in the io type for the scan
// (which consumes it as a 16-bit MFMA operand anyway) and once in the state type
// where the caller asked for it. The running sums of A v are taken in fp64, so
// the decay between two tokens is exact to fp32 however far into the chunk they
// lie. The state kernel feeds the matrix cores v x exp(...) as a sum of two
// 16-bit values (high part and rounding residual), which makes each product
// accurate to about 2^-16 instead of 2^-8; the scan rounds its operands once.
//
// MFMA operand layouts (gfx950, checked on the hardware):
//   16x16x32: lane l holds A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16],
//             j < 8; the result D[4 (l / 16) + i][l % 16], i < 4.
//   32x32x16: lane l holds A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32];
//             the result D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i < 16.
// Both operands want eight consecutive values of the contracted index per lane.
// Where that index is the token (state: sum over s; scan: sum over s), the
// token-major inputs are transposed on their way into LDS.
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
    int* list_head;       // workspace [nchunks]: first request whose last chunk is c
    int* list_next;       // workspace [batch]
    int64_t tokens, nchunks, batch;
    float dt_min, dt_max;
    int32_t nheads, ngroups, heads_per_group;
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

// Per chunk and head: the clamped step v_s and the inclusive running sum
// cum_s = sum_{j<=s} A v_j (fp64) for s < len, into LDS; zero past len. Every
// thread of the workgroup calls it; it ends with a barrier.
template <int Q>
__device__ __forceinline__ void chunk_steps(const SsdParams& p, const Chunk& ch, int h, float* sv,
                                            double* scum, double* swave) {
    static_assert(Q <= kThreads, "one step per thread");
    const int tid = threadIdx.x, lane = tid & 63;
    float v = 0.f;
    double a = 0.0;
    if (tid < ch.len) {
        float u = load_dt(p, (ch.lo + tid) * p.nheads + h);
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
    float* out = p.cb + (c * p.ngroups + g) * Q * Q;
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
                out[row * Q + sj * 32 + lane % 32] = acc[i];
            }
        }
    }
}

// ------------------------------------------------------------------- state

// Tokens staged per pass of the state kernel, and the LDS row pitch (in 16-bit
// elements) of the transposed tiles: 16 bytes of padding keeps rows 16-byte
// aligned for the fragment reads and staggers their banks.
constexpr int kStateBlock = 64;
constexpr int kPitch = kStateBlock + 8;

// LDS bytes of the state kernel: sv, scum, swave, sw, then x^T high and low
// parts [P][kPitch] and B^T [N][kPitch].
__host__ __device__ constexpr unsigned state_lds_bytes(int P, int N, int Q) {
    return 4u * Q + 8u * Q + 8u * kWaves + 4u * Q + 2u * (2 * P + N) * kPitch;
}

// One workgroup per (chunk, head); only the workgroups of chunks that open a
// request (the first chunk, or seq_idx changes) work: each walks its request's
// chunks in order with the state in MFMA accumulators. Wave w owns the
// accumulator tiles of dstate columns [w N/4, (w + 1) N/4) for every row p.
template <typename IT, typename ST, int P, int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(const SsdParams p) {
    typedef typename Mfma<IT>::v8 v8;
    constexpr int PT = P / 16;             // row tiles
    constexpr int NTW = N / 16 / kWaves;   // column tiles per wave
    static_assert(NTW >= 1 && P % 16 == 0, "tiles");
    const int64_t c0 = blockIdx.x / p.nheads;
    const int h = blockIdx.x % p.nheads;
    if (c0 > 0 && load_index(p.seq_idx, p.meta_i64, c0) == load_index(p.seq_idx, p.meta_i64, c0 - 1))
        return;
    const int g = h / p.heads_per_group;
    const int H = p.nheads;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sv = reinterpret_cast<float*>(smem);
    double* scum = reinterpret_cast<double*>(sv + Q);
    double* swave = scum + Q;
    float* sw = reinterpret_cast<float*>(swave + kWaves);
    unsigned short* xhi = reinterpret_cast<unsigned short*>(sw + Q);
    unsigned short* xlo = xhi + P * kPitch;
    unsigned short* bt = xlo + P * kPitch;

    // Accumulator tile (pt, j): rows p = 16 pt + 4 (lane / 16) + i, columns
    // n = 16 (wave NTW + j) + lane % 16.
    f32x4 acc[PT][NTW];
    const int64_t req = uniform64(load_index(p.seq_idx, p.meta_i64, c0));
    const bool has_init = p.init && req >= 0 && req < p.batch;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pr = 16 * pt + 4 * (lane / 16) + i;
                const int n = 16 * (wave * NTW + j) + lane % 16;
                acc[pt][j][i] =
                    has_init ? load_state<ST>(p.init, ((req * H + h) * P + pr) * N + n) : 0.f;
            }

    const IT* xp = static_cast<const IT*>(p.x);
    const IT* Bp = static_cast<const IT*>(p.B);
    for (int64_t c = c0; c < p.nchunks; ++c) {
        if (c > c0 && load_index(p.seq_idx, p.meta_i64, c) != load_index(p.seq_idx, p.meta_i64, c - 1))
            break;
        const Chunk ch = chunk_of<Q>(p, c);
        lds_barrier();  // the previous chunk is done with sv / scum / the tiles
        chunk_steps<Q>(p, ch, h, sv, scum, swave);
        if (ch.len > 0) {
            const double last = scum[ch.len - 1];
            if (tid < ch.len) sw[tid] = expf(static_cast<float>(last - scum[tid])) * sv[tid];
            const float decay = expf(static_cast<float>(last));
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[pt][j] *= decay;

            for (int s0 = 0; s0 < ch.len; s0 += kStateBlock) {
                lds_barrier();  // sw visible; the previous block's tiles consumed
                // x^T: thread (token pair jp, row octet q) -> rows 8q.., columns 2jp, 2jp+1.
                for (int idx = tid; idx < (kStateBlock / 2) * (P / 8); idx += kThreads) {
                    const int jp = idx % (kStateBlock / 2), q = idx / (kStateBlock / 2);
                    const int s = s0 + 2 * jp;
                    u16x8 r0 = {}, r1 = {};
                    float w0 = 0.f, w1 = 0.f;
                    if (s < ch.len) {
                        r0 = *reinterpret_cast<const u16x8*>(xp + ((ch.lo + s) * H + h) * P + 8 * q);
                        w0 = sw[s];
                    }
                    if (s + 1 < ch.len) {
                        r1 = *reinterpret_cast<const u16x8*>(xp + ((ch.lo + s + 1) * H + h) * P + 8 * q);
                        w1 = sw[s + 1];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float a0 = f32_of<IT>(r0[e]) * w0, a1 = f32_of<IT>(r1[e]) * w1;
                        const unsigned short h0 = bits_of<IT>(a0), h1 = bits_of<IT>(a1);
                        const unsigned short l0 = bits_of<IT>(a0 - f32_of<IT>(h0));
                        const unsigned short l1 = bits_of<IT>(a1 - f32_of<IT>(h1));
                        const int o = (8 * q + e) * kPitch + 2 * jp;
                        *reinterpret_cast<unsigned*>(xhi + o) = h0 | (static_cast<unsigned>(h1) << 16);
                        *reinterpret_cast<unsigned*>(xlo + o) = l0 | (static_cast<unsigned>(l1) << 16);
                    }
                }
                // B^T: thread (token pair, dstate octet) -> rows 8q.., columns 2jp, 2jp+1.
                for (int idx = tid; idx < (kStateBlock / 2) * (N / 8); idx += kThreads) {
                    const int jp = idx % (kStateBlock / 2), q = idx / (kStateBlock / 2);
                    const int s = s0 + 2 * jp;
                    u16x8 r0 = {}, r1 = {};
                    if (s < ch.len)
                        r0 = *reinterpret_cast<const u16x8*>(Bp + ((ch.lo + s) * p.ngroups + g) * N + 8 * q);
                    if (s + 1 < ch.len)
                        r1 = *reinterpret_cast<const u16x8*>(Bp + ((ch.lo + s + 1) * p.ngroups + g) * N + 8 * q);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        *reinterpret_cast<unsigned*>(bt + (8 * q + e) * kPitch + 2 * jp) =
                            r0[e] | (static_cast<unsigned>(r1[e]) << 16);
                }
                lds_barrier();
#pragma unroll
                for (int kk = 0; kk < kStateBlock; kk += 32) {
                    if (s0 + kk >= ch.len) break;
                    const int col = kk + 8 * (lane / 16);
                    v8 bf[NTW];
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
                        bf[j] = *reinterpret_cast<const v8*>(bt + (16 * (wave * NTW + j) + lane % 16) * kPitch + col);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const int row = (16 * pt + lane % 16) * kPitch + col;
                        const v8 ah = *reinterpret_cast<const v8*>(xhi + row);
                        const v8 al = *reinterpret_cast<const v8*>(xlo + row);
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            acc[pt][j] = Mfma<IT>::mma16(ah, bf[j], acc[pt][j]);
                            acc[pt][j] = Mfma<IT>::mma16(al, bf[j], acc[pt][j]);
                        }
                    }
                }
            }
        }
        // The state after chunk c: in the io type for the scan of chunk c + 1, and
        // in the state type where the caller asked for it.
        IT* s16 = static_cast<IT*>(p.s16);
        const bool feeds_next = c + 1 < p.nchunks &&
            load_index(p.seq_idx, p.meta_i64, c + 1) == load_index(p.seq_idx, p.meta_i64, c);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pr = 16 * pt + 4 * (lane / 16) + i;
                    const int n = 16 * (wave * NTW + j) + lane % 16;
                    const int64_t e = (static_cast<int64_t>(h) * P + pr) * N + n;
                    if (feeds_next) s16[c * H * P * N + e] = static_cast<IT>(acc[pt][j][i]);
                    if (p.return_all) store_state<ST>(p.states, c * H * P * N + e, acc[pt][j][i]);
                }
        if (!p.return_all) {
            int64_t b = uniform64(p.list_head[c]);
            for (int64_t hops = 0; b >= 0 && b < p.batch && hops < p.batch; ++hops) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int pr = 16 * pt + 4 * (lane / 16) + i;
                            const int n = 16 * (wave * NTW + j) + lane % 16;
                            store_state<ST>(p.states, ((b * H + h) * P + pr) * N + n, acc[pt][j][i]);
                        }
                b = uniform64(p.list_next[b]);
            }
        }
    }
}

// -------------------------------------------------------------------- scan

constexpr int scan_pitch(int Q) { return Q + 8; }

// LDS bytes of the scan kernel: sv, cum (fp32), scum (fp64), swave, then
// (v x)^T [P][Q + 8].
__host__ __device__ constexpr unsigned scan_lds_bytes(int P, int Q) {
    return 4u * Q + 4u * Q + 8u * Q + 8u * kWaves + 2u * P * scan_pitch(Q);
}

// One workgroup per (chunk, head). Wave w owns the output rows of token tiles
// w, w + 4, w + 8, ... (16 tokens each) for all P columns.
template <typename IT, typename ST, int P, int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(const SsdParams p) {
    typedef typename Mfma<IT>::v8 v8;
    constexpr int PT = P / 16;
    constexpr int TT = Q / 16 / kWaves;  // token tiles per wave
    constexpr int XP = scan_pitch(Q);
    const int64_t c = blockIdx.x / p.nheads;
    const int h = blockIdx.x % p.nheads;
    const Chunk ch = chunk_of<Q>(p, c);
    if (ch.len == 0) return;
    const int g = h / p.heads_per_group;
    const int H = p.nheads;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;

    extern __shared__ __align__(16) unsigned char smem[];
    float* sv = reinterpret_cast<float*>(smem);
    float* cumf = sv + Q;
    double* scum = reinterpret_cast<double*>(cumf + Q);
    double* swave = scum + Q;
    unsigned short* xv = reinterpret_cast<unsigned short*>(swave + kWaves);

    chunk_steps<Q>(p, ch, h, sv, scum, swave);
    if (tid < Q) cumf[tid] = static_cast<float>(scum[tid]);

    // (v x)^T into LDS, rounded once to the io type.
    const IT* xp = static_cast<const IT*>(p.x);
    for (int idx = tid; idx < (Q / 2) * (P / 8); idx += kThreads) {
        const int jp = idx % (Q / 2), q = idx / (Q / 2);
        const int s = 2 * jp;
        u16x8 r0 = {}, r1 = {};
        float v0 = 0.f, v1 = 0.f;
        if (s < ch.len) {
            r0 = *reinterpret_cast<const u16x8*>(xp + ((ch.lo + s) * H + h) * P + 8 * q);
            v0 = sv[s];
        }
        if (s + 1 < ch.len) {
            r1 = *reinterpret_cast<const u16x8*>(xp + ((ch.lo + s + 1) * H + h) * P + 8 * q);
            v1 = sv[s + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *reinterpret_cast<unsigned*>(xv + (8 * q + e) * XP + s) =
                bits_of<IT>(f32_of<IT>(r0[e]) * v0) |
                (static_cast<unsigned>(bits_of<IT>(f32_of<IT>(r1[e]) * v1)) << 16);
    }

    f32x4 acc[TT][PT];
#pragma unroll
    for (int k = 0; k < TT; ++k)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[k][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- the state entering the chunk: C_t . S_in, then scaled by exp(cum_t)
    const int64_t req = uniform64(load_index(p.seq_idx, p.meta_i64, c));
    const bool opens = c == 0 || req != load_index(p.seq_idx, p.meta_i64, c - 1);
    const bool from_init = opens && p.init && req >= 0 && req < p.batch;
    const IT* Cp = static_cast<const IT*>(p.C);
    if (!opens || from_init) {
#pragma unroll
        for (int kk = 0; kk < N; kk += 32) {
            const int col = kk + 8 * (lane / 16);
            v8 sf[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                if (!opens) {
                    sf[pt] = *reinterpret_cast<const v8*>(static_cast<const IT*>(p.s16) +
                                                          (((c - 1) * H + h) * P + pr) * N + col);
                } else {
                    const int64_t base = ((req * H + h) * P + pr) * N + col;
#pragma unroll
                    for (int j = 0; j < 8; ++j) sf[pt][j] = static_cast<IT>(load_state<ST>(p.init, base + j));
                }
            }
#pragma unroll
            for (int k = 0; k < TT; ++k) {
                const int t0 = 16 * (wave + kWaves * k);
                if (t0 >= ch.len) continue;
                const int t = min(t0 + lane % 16, ch.len - 1);
                const v8 ca = *reinterpret_cast<const v8*>(Cp + ((ch.lo + t) * p.ngroups + g) * N + col);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[k][pt] = Mfma<IT>::mma16(ca, sf[pt], acc[k][pt]);
            }
        }
#pragma unroll
        for (int k = 0; k < TT; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = min(16 * (wave + kWaves * k) + 4 * (lane / 16) + i, Q - 1);
                const float f = expf(static_cast<float>(scum[t]));
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) acc[k][pt][i] *= f;
            }
    }
    lds_barrier();  // (v x)^T and cumf complete

    // ---- inside the chunk: (CB masked by the decays) times (v x)
    const float* cbp = p.cb + (c * p.ngroups + g) * Q * Q;
    for (int kk = 0; kk < ch.len; kk += 32) {
        const int col = kk + 8 * (lane / 16);
        v8 xf[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            xf[pt] = *reinterpret_cast<const v8*>(xv + (16 * pt + lane % 16) * XP + col);
        float cs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cs[j] = cumf[col + j];
#pragma unroll
        for (int k = 0; k < TT; ++k) {
            const int t0 = 16 * (wave + kWaves * k);
            if (t0 >= ch.len || t0 + 15 < kk) continue;
            const int t = t0 + lane % 16;
            const f32x4* cbr = reinterpret_cast<const f32x4*>(cbp + t * Q + col);
            const f32x4 m0 = cbr[0], m1 = cbr[1];
            const float ct = cumf[t];
            v8 a;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float m = j < 4 ? m0[j] : m1[j - 4];
                const bool live = col + j <= t && t < ch.len;
                a[j] = static_cast<IT>(live ? m * expf(ct - cs[j]) : 0.f);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[k][pt] = Mfma<IT>::mma16(a, xf[pt], acc[k][pt]);
        }
    }

    // ---- skip term, gate, store
    const IT* zp = static_cast<const IT*>(p.z);
    IT* op = static_cast<IT*>(p.out);
#pragma unroll
    for (int k = 0; k < TT; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * (wave + kWaves * k) + 4 * (lane / 16) + i;
            if (t >= ch.len) continue;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int pr = 16 * pt + lane % 16;
                const int64_t xi = ((ch.lo + t) * H + h) * P + pr;
                float y = acc[k][pt][i];
                if (p.D) y += (p.D_per_dim ? p.D[h * P + pr] : p.D[h]) * static_cast<float>(xp[xi]);
                if (zp) y *= silu_f32(static_cast<float>(zp[xi]));
                op[xi] = static_cast<IT>(y);
            }
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
    const dim3 grid(static_cast<unsigned>(p.nchunks * p.nheads));
    hipLaunchKernelGGL((ssd_state_kernel<IT, ST, P, N, Q>), grid, dim3(kThreads),
                       state_lds_bytes(P, N, Q), stream, p);
    hipLaunchKernelGGL((ssd_scan_kernel<IT, ST, P, N, Q>), grid, dim3(kThreads), scan_lds_bytes(P, Q),
                       stream, p);
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
