// ssu_kernel.hpp -- the selective state update kernel for gfx950 (CDNA4, wave64).
//
// One workgroup owns a (sequence, block of heads of one group, block of rows)
// tile. Each head of the block gets a head group of HW wave64s (four, or one or
// two for dstate rows of 64 bytes or less). The head's rows are spread so that
// one vector-memory instruction of a wave covers RPI whole consecutive dstate
// rows -- 64 lanes x 16 bytes, one contiguous run of the slot -- and each lane
// owns the same VEC consecutive dstate elements of RL different rows for the
// whole call. The state therefore crosses HBM
// exactly once in each direction: read once per sequence, kept in fp32 registers
// across all tokens of a packed sequence, written once per token.
//
// The per-token operands shared along a row (B and C of the group, N values
// each) or along dstate (x, z, dt of the head, one per row) are staged in LDS
// once per workgroup, already widened to fp32 and turned into the per-row
// factors the update needs (v*x, exp(A*v), D*x, z*sigmoid(z)); B and C serve all
// heads of the workgroup. A packed sequence stages up to kStageTokens tokens at a
// time, so its token loop runs without a barrier or a global load: one barrier
// per chunk of tokens. The dot product over dstate is a lane-local FMA chain plus
// a cross-lane sum over the LPR lanes of a row (DPP quad/mirror moves inside
// 16-lane rows, one permute across rows when LPR > 16); the first lane of each
// row then finishes that row (skip term, gate, rounding) and stores it.
//
// Memory ordering: gfx9 counts loads and stores in one vmcnt queue, so every load
// the next step waits for is issued before anything it must not wait for: the
// staged operands are requested before the state. Workgroup barriers fence LDS
// only, so the state loads stay in flight across them.
//
// Semantics follow include/ssu.h.
#pragma once

#include <hip/hip_runtime.h>

#include "ssu_launch.h"

namespace ssu {

// ---------------------------------------------------------------- storage types

template <int W>
struct Words {
    typedef unsigned type __attribute__((ext_vector_type(W)));
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Widen / narrow one 32-bit word of a storage type.
template <typename T>
struct Pack;

template <>
struct Pack<float> {
    static constexpr int kPerWord = 1;
    __device__ static void widen(unsigned w, float* f) { f[0] = __uint_as_float(w); }
    __device__ static unsigned narrow(const float* f) { return __float_as_uint(f[0]); }
};

template <>
struct Pack<__bf16> {
    static constexpr int kPerWord = 2;
    __device__ static void widen(unsigned w, float* f) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xffff0000u);
    }
    __device__ static unsigned narrow(const float* f) {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    }
};

template <>
struct Pack<_Float16> {
    static constexpr int kPerWord = 2;
    __device__ static void widen(unsigned w, float* f) {
        f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        f[0] = v.x;
        f[1] = v.y;
    }
    __device__ static unsigned narrow(const float* f) {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
    }
};

// Bit pattern of an io element. Staged operands are held as bits so that the
// compiler cannot widen them next to their load (which would wait for it).
template <typename T> struct Bits { typedef unsigned short type; };
template <> struct Bits<float> { typedef unsigned type; };

template <typename T>
__device__ __forceinline__ float widen_io(typename Bits<T>::type b) {
    return static_cast<float>(__builtin_bit_cast(T, b));
}

template <typename T>
__device__ __forceinline__ void store_io(void* p, int64_t i, float v) {
    static_cast<T*>(p)[i] = static_cast<T>(v);
}

__device__ __forceinline__ int64_t load_index(const void* p, int is64, int64_t i) {
    return is64 ? static_cast<const int64_t*>(p)[i]
                : static_cast<int64_t>(static_cast<const int32_t*>(p)[i]);
}

// Make a value the compiler cannot prove uniform live in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
    const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Workgroup barrier that orders LDS only; outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR consecutive lanes; every lane gets its group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(LPR >= 2 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "LPR");
    v += dpp<0xB1>(v);                            // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPR >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8) v += dpp<0x141>(v);   // row_half_mirror: quads of an 8
    if constexpr (LPR >= 16) v += dpp<0x140>(v);  // row_mirror: halves of a 16
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

// ------------------------------------------------------- stochastic rounding

// Philox4x32 (Salmon, Moraes, Dror, Shaw, SC'11): per round, the products of
// counter words 0 and 2 with the two multipliers; high halves are mixed with the
// other counter words and the key, low halves pass through; the key steps by the
// two Weyl increments between rounds.
__device__ __forceinline__ void philox4x32_rounds(uint32_t (&c)[4], uint32_t k0, uint32_t k1,
                                                  int rounds) {
#pragma unroll 10
    for (int r = 0; r < rounds; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // One 32x32->64 multiply-add each (v_mad_u64_u32) gives both halves.
        const uint64_t p0 = static_cast<uint64_t>(c[0]) * 0xD2511F53u;
        const uint64_t p1 = static_cast<uint64_t>(c[2]) * 0xCD9E8D57u;
        const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = static_cast<uint32_t>(p1);
        c[2] = n2;
        c[3] = static_cast<uint32_t>(p0);
    }
}

// The round count is a run-time value; the common 10 gets a fully unrolled copy.
__device__ __forceinline__ void philox4x32(uint32_t (&c)[4], uint32_t k0, uint32_t k1,
                                           int rounds) {
    if (rounds == 10)
        philox4x32_rounds(c, k0, k1, 10);
    else
        philox4x32_rounds(c, k0, k1, rounds);
}

// A power of two 2^k for k in [-126, 127], exactly.
__device__ __forceinline__ float pow2f(int k) {
    return __uint_as_float(static_cast<unsigned>(127 + k) << 23);
}

// Stochastic rounding of v with random word w (its top bits used), as 16-bit
// patterns. bf16: adding the word's top 16 bits below the bf16 mantissa and
// truncating rounds away from zero exactly when U >= 1 - frac (U = those bits /
// 2^16).
__device__ __forceinline__ unsigned sr_bits_bf16(float v, uint32_t w) {
    const unsigned u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u)  // inf, nan: plain conversion
        return __builtin_bit_cast(unsigned short, static_cast<__bf16>(v));
    return (u + (w >> 16)) >> 16;
}

// fp16: by exact power-of-two scaling to the fp16 spacing at |v| (normals share
// exponent -14 with the subnormals below them); the threshold U >= 1 - frac is
// decided as the sign of (U - 1) + frac, which rounding cannot change.
__device__ __forceinline__ unsigned sr_bits_f16(float v, uint32_t w) {
    const float a = fabsf(v);
    if (!(a < __builtin_inff()) || a == 0.f)
        return __builtin_bit_cast(unsigned short, static_cast<_Float16>(v));
    const int e = static_cast<int>(__float_as_uint(a) >> 23) - 127;
    const int qexp = (e > -14 ? e : -14) - 10;
    const float t = a * pow2f(-qexp);
    const float m = floorf(t);
    const float frac = t - m;
    const float U = static_cast<float>(w >> 8) * pow2f(-24);
    float r = (m + (((U - 1.f) + frac >= 0.f) ? 1.f : 0.f)) * pow2f(qexp);
    if (r > 65504.f) r = __builtin_inff();
    return __builtin_bit_cast(unsigned short, static_cast<_Float16>(copysignf(r, v)));
}

// ------------------------------------------------------------------- math

__device__ __forceinline__ float softplus_f32(float v) {
    return v > 0.f ? v + log1pf(expf(-v)) : log1pf(expf(v));
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.f + expf(-z)); }

__device__ __forceinline__ bool slot_ok(int64_t s, const KernelParams& p) {
    return s != p.pad_slot_id && s >= 0 && s < p.nslots;
}

// Tokens of a packed sequence staged in LDS at a time.
constexpr int kStageTokens = 8;

// LDS floats one staged token takes: B and C of the group, then four per-row
// factors for every row of every head of the workgroup.
__host__ __device__ constexpr int token_floats(int dstate, int heads_per_block, int rows) {
    return 2 * dstate + 4 * heads_per_block * rows;
}

// LDS bytes of a launch: `tokens` staged tokens, their destination ids, and one
// row sum per row of the workgroup (each wave's rows, for its coalesced store).
__host__ __device__ constexpr unsigned lds_bytes(int dstate, int heads_per_block, int rows,
                                                 int tokens) {
    return tokens * (4u * token_floats(dstate, heads_per_block, rows) + 8u) +
           4u * heads_per_block * rows;
}

// Order this wave's earlier LDS writes before its later LDS reads (other lanes).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Lane geometry of one (state dtype, dstate, load depth) instance. Every lane
// load moves 16 bytes. A head group of HW waves covers RB consecutive rows of
// one head. Rows of more than 64 bytes take four waves per head group, each lane
// up to LOADS rows (at most a quarter of a row's lanes, so RB stays within 64
// rows). Rows of 64 bytes or less (dstate 16, or 32 with a 16-bit state) give a
// lane LOADS rows, or all a row's lanes' worth if fewer, and the head group only
// as many waves as it takes to cover 64 rows: one or two, so that each lane keeps
// 32-64 bytes in flight instead of one short load.
template <typename ST, int N, int LOADS>
struct Geometry {
    static constexpr int kMaxVec = 16 / static_cast<int>(sizeof(ST));
    static constexpr int VEC = kMaxVec;                // elements per lane-load
    static constexpr int LPR = N / VEC;                // lanes per dstate row
    static constexpr int RPI = 64 / LPR;               // rows per wave instruction
    static constexpr bool kShortRows = N * static_cast<int>(sizeof(ST)) <= 64;
    static constexpr int RL = kShortRows ? (LOADS < LPR ? LOADS : LPR)
                                         : (LOADS < LPR / 4 ? LOADS : LPR / 4);  // loads per lane
    static constexpr int HW = kShortRows ? 64 / (RPI * RL) : 4;  // waves per head group
    static constexpr int HT = 64 * HW;                          // threads per head group
    static constexpr int RB = HW * RPI * RL;                    // rows per head group
    static_assert(N % VEC == 0 && LPR >= 2, "a row spans at least two lanes");
    static_assert(RL >= 1 && HW >= 1 && HW <= 4 && RPI * RL <= 64 && RB <= 64, "geometry");
};

// Tile of workgroup `id` out of `n` when each XCD should walk a contiguous range
// of tiles: workgroup id lands on XCD id % kXcds, and the XCDs that receive one
// extra workgroup come first. A bijection of [0, n).
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t n) {
    const int64_t xcd = id % kXcds, k = id / kXcds;
    const int64_t per = (n + kXcds - 1) / kXcds;
    int64_t tall = n % kXcds;
    if (tall == 0) tall = kXcds;
    return xcd < tall ? xcd * per + k : tall * per + (xcd - tall) * (per - 1) + k;
}

// Tile of workgroup `id` out of `n` = sequences x `per_seq` tiles when every XCD
// should take an equal contiguous share of each sequence's tiles (a block of its
// heads): XCD x walks, sequence after sequence, tiles [x per_seq / kXcds,
// (x + 1) per_seq / kXcds) of each. Every XCD then carries the same share of
// every sequence, however the sequences' token counts differ, and still streams
// contiguous memory. A bijection of [0, n) when per_seq is a multiple of kXcds
// (else the contiguous-range order).
__device__ __forceinline__ int64_t xcd_split(int64_t id, int64_t n, int64_t per_seq) {
    if (per_seq % kXcds) return xcd_tile(id, n);
    const int64_t share = per_seq / kXcds;
    const int64_t xcd = id % kXcds, k = id / kXcds;
    return (k / share) * per_seq + xcd * share + k % share;
}

// ------------------------------------------------------------------ kernel

template <typename ST, typename IT, int N, int LOADS, bool PACKED, bool SR>
__global__ __launch_bounds__((Geometry<ST, N, LOADS>::HT * max_heads_per_block(N, PACKED))) void ssu_update_kernel(
    const KernelParams p) {
    // Lane geometry.
    typedef Geometry<ST, N, LOADS> Geo;
    constexpr int VEC = Geo::VEC, LPR = Geo::LPR, RPI = Geo::RPI, RL = Geo::RL, RB = Geo::RB;
    constexpr int HT = Geo::HT, HW = Geo::HW;
    constexpr int W = VEC / Pack<ST>::kPerWord;               // 32-bit words per lane-load
    constexpr int T = PACKED ? kStageTokens : 1;              // tokens staged at a time
    typedef typename Words<W>::type words_t;

    const int tid = threadIdx.x;
    // Head within the workgroup and wave within the head group are wave-uniform;
    // saying so keeps the slot base addresses in scalar registers.
    const int lh = __builtin_amdgcn_readfirstlane(tid / HT);
    const int ht = tid % HT;                 // thread within the head group
    const int wave = __builtin_amdgcn_readfirstlane(ht / 64);
    const int lane = ht % 64;
    const int rg = lane / LPR;               // row within one wave instruction
    const int n0 = (lane % LPR) * VEC;       // first dstate element of this lane
    const bool row_leader = (lane % LPR) == 0;

    int64_t wg = blockIdx.x;
    if (p.xcd_order == 1)
        wg = xcd_tile(wg, gridDim.x);
    else if (p.xcd_order == 2)
        wg = xcd_split(wg, gridDim.x, static_cast<int64_t>(p.head_blocks) * p.row_blocks);
    const int rb = static_cast<int>(wg % p.row_blocks);
    wg /= p.row_blocks;
    const int hblk = static_cast<int>(wg % p.head_blocks);
    const int64_t seq = wg / p.head_blocks;
    const int hpb = p.heads_per_block;
    const int h = hblk * hpb + lh;
    const int g = (hblk * hpb) / p.heads_per_group;
    const int H = p.nheads, P = p.headdim;

    // LDS: per staged token tt, B[N] C[N] then factors [4][hpb][RB]; after all
    // tokens, their destination ids.
    extern __shared__ float lds[];
    const int tok = token_floats(N, hpb, RB);
    int64_t* const sW = reinterpret_cast<int64_t*>(lds + T * tok);
    // This wave's row sums, indexed by row within the wave's RPI * RL rows.
    constexpr int WROWS = RPI * RL;
    float* const sY = reinterpret_cast<float*>(sW + T) + (lh * HW + wave) * WROWS;
    enum { kXV = 0, kDA = 1, kDX = 2, kGZ = 3 };  // v*x, exp(A*v), D*x, z*sigmoid(z)
    auto factor = [&](int tt, int which, int pl) -> float& {
        return lds[tt * tok + 2 * N + (which * hpb + lh) * RB + pl];
    };

    // ---- slot resolution (uniform across the workgroup)
    int64_t begin, len, r;
    if constexpr (PACKED) {
        if (p.cu) {
            const int64_t b0 = load_index(p.cu, p.meta_i64, seq);
            const int64_t b1 = load_index(p.cu, p.meta_i64, seq + 1);
            begin = uniform64(b0);
            len = uniform64(b1 - b0);
        } else {
            begin = seq * p.seq_len;
            len = p.seq_len;
        }
        if (begin < 0 || begin + len > p.rows || len <= 0) return;
        if (p.src) {
            const int64_t k = uniform64(p.na ? load_index(p.na, p.meta_i64, seq) : 1);
            if (k < 1 || k > p.steps) return;
            r = load_index(p.src, p.src_i64, seq * p.src_seq_stride + (k - 1) * p.src_step_stride);
        } else {
            r = seq;
        }
    } else {
        begin = seq;
        len = 1;
        r = p.src ? load_index(p.src, p.src_i64, seq) : seq;
    }
    r = uniform64(r);
    if (!slot_ok(r, p)) return;

    // ---- per-head constants
    uint32_t key0 = 0, key1 = 0;
    if constexpr (SR) {
        const uint64_t seed = static_cast<uint64_t>(uniform64(*p.rand_seed));
        key0 = static_cast<uint32_t>(seed);
        key1 = static_cast<uint32_t>(seed >> 32);
    }
    const float a_h = p.A[h];
    const float d_h = p.D ? p.D[h] : 0.f;
    const float bias_h = p.dt_bias ? p.dt_bias[h] : 0.f;
    const bool gated = p.z != nullptr;

    // ---- operand staging: raw loads into registers, factors into LDS once the
    // loads land. A chunk of nt tokens is spread over the workgroup: row factors
    // over (token, row) pairs of each head group, B/C over (token, n) pairs of the
    // whole workgroup, destination ids over the first nt threads. Elements past
    // the chunk or past headdim load a valid dummy address instead of branching.
    constexpr int ROW_PASSES = (T * RB + HT - 1) / HT;
    constexpr int BC_PASSES = (T * N + HT - 1) / HT;
    const int nthreads = HT * hpb;
    typedef typename Bits<IT>::type bits_t;
    const bits_t* const xp = static_cast<const bits_t*>(p.x);
    const bits_t* const zp = static_cast<const bits_t*>(gated ? p.z : p.x);  // ungated: unused
    const bits_t* const Bp = static_cast<const bits_t*>(p.B);
    const bits_t* const Cp = static_cast<const bits_t*>(p.C);
    struct RowStage {
        bits_t x, z;
        float dt;
    };
    RowStage rs[ROW_PASSES];
    bits_t bs[BC_PASSES], cs[BC_PASSES];
    int64_t dw = 0;
    // Raw destination slot of token t (validated where it is used).
    auto dest_load = [&](int64_t t) -> int64_t {
        if constexpr (PACKED) {
            if (p.dst)
                return t < p.steps
                           ? load_index(p.dst, p.dst_i64, seq * p.dst_seq_stride + t * p.dst_step_stride)
                           : p.pad_slot_id;
            return t == len - 1 ? r : p.pad_slot_id;
        } else {
            return p.dst ? load_index(p.dst, p.dst_i64, seq) : r;
        }
    };
    auto load_chunk = [&](int64_t t0, int64_t nt) {
#pragma unroll
        for (int q = 0; q < ROW_PASSES; ++q) {
            const int idx = ht + q * HT, k = idx / RB, pl = idx % RB;
            const bool live = k < nt && rb * RB + pl < P;
            const int64_t row = begin + t0 + k;
            const int64_t xi = live ? (row * H + h) * P + rb * RB + pl : 0;
            rs[q].x = xp[xi];
            rs[q].z = zp[xi];
            rs[q].dt = p.dt[p.dt_per_dim ? xi : (live ? row * H + h : 0)];
        }
#pragma unroll
        for (int q = 0; q < BC_PASSES; ++q) {
            const int idx = tid + q * nthreads, k = idx / N, n = idx % N;
            const int64_t bi = k < nt ? ((begin + t0 + k) * p.ngroups + g) * N + n : 0;
            bs[q] = Bp[bi];
            cs[q] = Cp[bi];
        }
        if (tid < nt) dw = dest_load(t0 + tid);
    };
    auto store_chunk = [&](int64_t nt) {
#pragma unroll
        for (int q = 0; q < ROW_PASSES; ++q) {
            const int idx = ht + q * HT, k = idx / RB, pl = idx % RB;
            if (k < nt) {
                float xv = 0.f, dA = 0.f, dx = 0.f, gz = 1.f;
                if (rb * RB + pl < P) {
                    const float x = widen_io<IT>(rs[q].x);
                    float v = rs[q].dt + bias_h;
                    if (p.dt_softplus) v = softplus_f32(v);
                    dA = expf(a_h * v);
                    xv = v * x;
                    dx = d_h * x;
                    if (gated) gz = silu_f32(widen_io<IT>(rs[q].z));
                }
                factor(k, kXV, pl) = xv;
                factor(k, kDA, pl) = dA;
                factor(k, kDX, pl) = dx;
                factor(k, kGZ, pl) = gz;
            }
        }
#pragma unroll
        for (int q = 0; q < BC_PASSES; ++q) {
            const int idx = tid + q * nthreads, k = idx / N, n = idx % N;
            if (k < nt) {
                lds[k * tok + n] = widen_io<IT>(bs[q]);
                lds[k * tok + N + n] = widen_io<IT>(cs[q]);
            }
        }
        if (tid < nt) sW[tid] = dw;
    };

    // The first chunk's operands are requested before the state, so waiting for
    // them does not wait for the state.
    const int64_t first = len < T ? len : T;
    load_chunk(0, first);

    // ---- state gather: RL row-loads per lane, all in flight at once. Rows past
    // headdim (a ragged last block) read the last row instead and are never stored.
    const size_t slot_bytes = static_cast<size_t>(H) * P * N * sizeof(ST);
    const size_t head_bytes = static_cast<size_t>(P) * N * sizeof(ST);
    const bool full_block = rb * RB + RB <= P;
    int prow_of[RL];
    unsigned off[RL];
#pragma unroll
    for (int i = 0; i < RL; ++i) {
        prow_of[i] = rb * RB + wave * (RPI * RL) + i * RPI + rg;
        const int pr = prow_of[i] < P ? prow_of[i] : P - 1;
        off[i] = (static_cast<unsigned>(pr) * N + n0) * sizeof(ST);
    }
    words_t raw[RL];
    {
        const char* tile = static_cast<const char*>(p.state) + r * slot_bytes + h * head_bytes;
#pragma unroll
        for (int i = 0; i < RL; ++i)
            raw[i] = __builtin_nontemporal_load(reinterpret_cast<const words_t*>(tile + off[i]));
    }

    store_chunk(first);
    lds_barrier();

    float s[RL][VEC];
#pragma unroll
    for (int i = 0; i < RL; ++i)
#pragma unroll
        for (int k = 0; k < W; ++k) Pack<ST>::widen(raw[i][k], &s[i][k * Pack<ST>::kPerWord]);

    char* const head_base = static_cast<char*>(p.state) + h * head_bytes;
    for (int64_t t = 0; t < len; ++t) {
        int tt = 0;
        if constexpr (PACKED) {
            tt = static_cast<int>(t % T);
            if (t > 0 && tt == 0) {
                // Next chunk: every wave is done with the previous one first.
                lds_barrier();
                const int64_t nt = len - t < T ? len - t : T;
                load_chunk(t, nt);
                store_chunk(nt);
                lds_barrier();
            }
        }
        const float* const sB = lds + tt * tok;
        const float* const sC = sB + N;
        float bv[VEC], cv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            bv[e] = sB[n0 + e];
            cv[e] = sC[n0 + e];
        }
        const int64_t out_row = ((begin + t) * H + h) * P;
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int pl = prow_of[i] - rb * RB;
            const float dA = factor(tt, kDA, pl);
            const float xv = factor(tt, kXV, pl);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s[i][e] = fmaf(s[i][e], dA, xv * bv[e]);
                acc = fmaf(s[i][e], cv[e], acc);
            }
            acc = group_sum<LPR>(acc);
            if (row_leader) sY[i * RPI + rg] = acc;
        }
        // The wave's rows are contiguous: lane k finishes row k (skip term, gate,
        // rounding) so that `out` leaves in one coalesced store.
        wave_lds_sync();
        {
            const int wrow0 = wave * WROWS;
            const int prow_k = rb * RB + wrow0 + lane;
            if (lane < WROWS && prow_k < P) {
                const float y = (sY[lane] + factor(tt, kDX, wrow0 + lane)) *
                                factor(tt, kGZ, wrow0 + lane);
                store_io<IT>(p.out, out_row + prow_k, y);
            }
        }
        wave_lds_sync();  // the next token's row sums reuse sY

        // ---- state scatter for this token
        const int64_t w = uniform64(sW[tt]);
        if (!p.disable_state_update && slot_ok(w, p)) {
            char* tile = head_base + w * slot_bytes;
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                words_t o;
                if constexpr (SR) {
                    // Random bits for this lane's VEC elements e0 .. e0 + VEC - 1:
                    // fp16 takes the top 24 bits of word e % 4 of Philox(e / 4, row);
                    // bf16 the low / high half (even / odd e) of word (e % 8) / 2 of
                    // Philox(e / 8, row).
                    const int64_t row = begin + t;
                    const uint32_t rlo = static_cast<uint32_t>(row);
                    const uint32_t rhi = static_cast<uint32_t>(static_cast<uint64_t>(row) >> 32);
                    const uint32_t e0 =
                        static_cast<uint32_t>((static_cast<int64_t>(h) * P + prow_of[i]) * N + n0);
                    unsigned half[VEC];
                    if constexpr (__is_same(ST, __bf16)) {
                        // A lane's eight elements start at a multiple of 8: one call.
                        static_assert(VEC == 8, "eight bf16 elements per lane-load");
                        uint32_t c[4] = {e0 / 8, rlo, rhi, 0u};
                        philox4x32(c, key0, key1, p.philox_rounds);
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const uint32_t word = c[k / 2];
                            const uint32_t bits = (k & 1) ? (word >> 16) : (word & 0xFFFFu);
                            half[k] = sr_bits_bf16(s[i][k], bits << 16);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < VEC / 4; ++j) {
                            uint32_t c[4] = {e0 / 4 + j, rlo, rhi, 0u};
                            philox4x32(c, key0, key1, p.philox_rounds);
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                half[4 * j + k] = sr_bits_f16(s[i][4 * j + k], c[k]);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < W; ++k) o[k] = half[2 * k] | (half[2 * k + 1] << 16);
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k)
                        o[k] = Pack<ST>::narrow(&s[i][k * Pack<ST>::kPerWord]);
                }
                if (full_block || prow_of[i] < P)
                    __builtin_nontemporal_store(o, reinterpret_cast<words_t*>(tile + off[i]));
            }
        }
    }
}

// ---------------------------------------------------------------- launchers

template <typename ST, typename IT, int N, int LOADS>
hipError_t launch_instance(KernelParams p, int64_t nseq, hipStream_t stream, LaunchShape* shape) {
    typedef Geometry<ST, N, LOADS> Geo;
    constexpr int RB = Geo::RB;
    p.row_blocks = (p.headdim + RB - 1) / RB;
    const uint64_t blocks = static_cast<uint64_t>(nseq) * p.head_blocks * p.row_blocks;
    if (blocks > 0x7fffffffull) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks));
    const dim3 block(static_cast<unsigned>(Geo::HT * p.heads_per_block));
    const unsigned lds = lds_bytes(N, p.heads_per_block, RB, p.packed ? kStageTokens : 1);
    if (shape) *shape = LaunchShape{grid.x, block.x, lds, static_cast<unsigned>(RB)};
    if constexpr (sizeof(ST) == 2) {
        if (p.rand_seed) {
            if (p.packed)
                hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, LOADS, true, true>), grid, block,
                                   lds, stream, p);
            else
                hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, LOADS, false, true>), grid,
                                   block, lds, stream, p);
            return hipGetLastError();
        }
    }
    if (p.packed)
        hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, LOADS, true, false>), grid, block, lds,
                           stream, p);
    else
        hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, LOADS, false, false>), grid, block, lds,
                           stream, p);
    return hipGetLastError();
}

template <typename ST, typename IT, int N>
hipError_t launch_depth(const KernelParams& p, int64_t nseq, hipStream_t stream,
                        LaunchShape* shape) {
    switch (p.loads_per_lane) {
        case 2: return launch_instance<ST, IT, N, 2>(p, nseq, stream, shape);
        case 4: return launch_instance<ST, IT, N, 4>(p, nseq, stream, shape);
        default: return hipErrorInvalidValue;
    }
}

template <typename ST, typename IT>
hipError_t launch_dstate(const KernelParams& p, int dstate, int64_t nseq, hipStream_t stream,
                         LaunchShape* shape) {
    switch (dstate) {
        case 16: return launch_depth<ST, IT, 16>(p, nseq, stream, shape);
        case 32: return launch_depth<ST, IT, 32>(p, nseq, stream, shape);
        case 64: return launch_depth<ST, IT, 64>(p, nseq, stream, shape);
        case 128: return launch_depth<ST, IT, 128>(p, nseq, stream, shape);
        case 256: return launch_depth<ST, IT, 256>(p, nseq, stream, shape);
        default: return hipErrorInvalidValue;
    }
}

// io dtype codes follow ssu_dtype: 0 fp32, 1 fp16, 2 bf16.
template <typename ST>
hipError_t launch_state(const KernelParams& p, int io_dtype, int dstate, int64_t nseq,
                        hipStream_t stream, LaunchShape* shape) {
    switch (io_dtype) {
        case 0: return launch_dstate<ST, float>(p, dstate, nseq, stream, shape);
        case 1: return launch_dstate<ST, _Float16>(p, dstate, nseq, stream, shape);
        case 2: return launch_dstate<ST, __bf16>(p, dstate, nseq, stream, shape);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
