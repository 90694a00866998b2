// ssu_kernel.hpp -- the selective state update kernel for gfx950 (CDNA4, wave64).
//
// One workgroup owns a (sequence, block of heads of one group, block of 64 rows)
// tile. Each head of the block gets a 256-thread head group (four wave64s). The
// head's rows are spread so that one vector-memory instruction of a wave covers
// RPI whole consecutive dstate rows -- 64 lanes x (16 or 8) bytes, one contiguous
// 1 KiB (or 512 B) run of the slot -- and each lane owns the same VEC consecutive
// dstate elements of RL different rows for the whole call. The state therefore
// crosses HBM exactly once in each direction: read once per sequence, kept in fp32
// registers across all tokens of a packed sequence, written once per token.
//
// Per token, the operands that are shared along a row (B and C of the group, N
// values each) or along dstate (x, z, dt of the head, one per row) are staged once
// in LDS, widened to fp32 and with dt -> v -> dA evaluated there, then read by
// every lane that needs them; B and C are shared by all heads of the workgroup.
// The dot product over dstate is a lane-local FMA chain followed by a cross-lane
// reduction over the LPR lanes of a row (DPP quad/mirror moves inside 16-lane
// rows, one permute across rows when LPR > 16). The per-row epilogue (D * x,
// SiLU gate, rounding, store of `out`) runs on one lane per row after the partial
// sums meet in LDS.
//
// Memory ordering: gfx9 counts loads and stores in one vmcnt queue, so every load
// the next step waits for is issued before anything it must not wait for. The
// token-0 operands are requested before the state, and token t+1's operands
// before token t's state stores. Workgroup barriers fence LDS only, so the state
// loads stay in flight across them. Stage buffers alternate between tokens.
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

// ------------------------------------------------------------------- math

__device__ __forceinline__ float softplus_f32(float v) {
    return v > 0.f ? v + log1pf(expf(-v)) : log1pf(expf(v));
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.f + expf(-z)); }

__device__ __forceinline__ bool slot_ok(int64_t s, const KernelParams& p) {
    return s != p.pad_slot_id && s >= 0 && s < p.nslots;
}

// Number of LDS floats a launch needs (double-buffered stage).
__host__ __device__ constexpr int lds_floats(int dstate, int heads_per_block) {
    return 2 * (2 * dstate + 5 * heads_per_block * kRowsPerBlock);
}

// ------------------------------------------------------------------ kernel

template <typename ST, typename IT, int N, bool PACKED>
__global__ __launch_bounds__(kHeadThreads* max_heads_per_block(N)) void ssu_update_kernel(
    const KernelParams p) {
    // Lane geometry.
    constexpr int kMaxVec = 16 / static_cast<int>(sizeof(ST));
    constexpr int VEC = kMaxVec < N / 4 ? kMaxVec : N / 4;    // elements per lane-load
    constexpr int W = VEC / Pack<ST>::kPerWord;               // 32-bit words per lane-load
    constexpr int LPR = N / VEC;                              // lanes per dstate row
    constexpr int RPI = 64 / LPR;                             // rows per wave instruction
    constexpr int RL = LPR / 4;                               // row-loads per lane
    constexpr int RB = kRowsPerBlock;
    static_assert(4 * RPI * RL == RB, "a head group covers one row block");
    typedef typename Words<W>::type words_t;

    extern __shared__ float lds[];
    const int hpb = p.heads_per_block;
    float* const sB = lds;                   // [2][N]
    float* const sC = sB + 2 * N;            // [2][N]
    float* const sRow = sC + 2 * N;          // [2][5][hpb][RB]: xv, dA, x, z, y
    enum { kXV = 0, kDA = 1, kX = 2, kZ = 3, kY = 4 };

    const int tid = threadIdx.x;
    // Head within the workgroup and wave within the head group are wave-uniform;
    // saying so keeps the slot base addresses in scalar registers.
    const int lh = __builtin_amdgcn_readfirstlane(tid / kHeadThreads);
    const int ht = tid % kHeadThreads;       // thread within the head group
    const int wave = __builtin_amdgcn_readfirstlane(ht / 64);
    const int lane = ht % 64;
    const int rg = lane / LPR;               // row within one wave instruction
    const int n0 = (lane % LPR) * VEC;       // first dstate element of this lane

    int64_t wg = blockIdx.x;
    const int rb = static_cast<int>(wg % p.row_blocks);
    wg /= p.row_blocks;
    const int hblk = static_cast<int>(wg % p.head_blocks);
    const int64_t seq = wg / p.head_blocks;
    const int h = hblk * hpb + lh;
    const int g = (hblk * hpb) / p.heads_per_group;
    const int H = p.nheads, P = p.headdim;
    auto row_slot = [&](int buf, int which, int pl) -> float& {
        return sRow[((buf * 5 + which) * hpb + lh) * RB + pl];
    };

    // ---- slot resolution (uniform across the workgroup)
    int64_t begin, len, r;
    if constexpr (PACKED) {
        const int64_t b0 = load_index(p.cu, p.meta_i64, seq);
        const int64_t b1 = load_index(p.cu, p.meta_i64, seq + 1);
        begin = uniform64(b0);
        len = uniform64(b1 - b0);
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
    const float a_h = p.A[h];
    const float d_h = p.D ? p.D[h] : 0.f;
    const float bias_h = p.dt_bias ? p.dt_bias[h] : 0.f;

    // ---- per-token operand staging: raw loads into registers, widened and written
    // to LDS only when the next step needs them. Threads that stage nothing load a
    // valid dummy address instead of branching.
    const int prow = rb * RB + ht;            // row this thread stages (ht < RB)
    const bool stages_row = ht < RB && prow < P;
    const bool stages_bc = tid < N;
    typedef typename Bits<IT>::type bits_t;
    const bits_t* const xp = static_cast<const bits_t*>(p.x);
    const bits_t* const zp = static_cast<const bits_t*>(p.z ? p.z : p.x);  // no gate: unused
    const bits_t* const Bp = static_cast<const bits_t*>(p.B);
    const bits_t* const Cp = static_cast<const bits_t*>(p.C);
    struct Stage {
        bits_t x, z, b, c;
        float dt;
        int64_t w;                             // raw destination id (validated at use)
    };
    auto stage_load = [&](int64_t t) -> Stage {
        Stage s;
        const int64_t row = begin + t;
        const int64_t xi = stages_row ? (row * H + h) * P + prow : 0;
        s.x = xp[xi];
        s.z = zp[xi];
        s.dt = p.dt[p.dt_per_dim ? xi : (stages_row ? row * H + h : 0)];
        const int64_t bi = stages_bc ? (row * p.ngroups + g) * N + tid : 0;
        s.b = Bp[bi];
        s.c = Cp[bi];
        if constexpr (PACKED) {
            if (p.dst)
                s.w = t < p.steps ? load_index(p.dst, p.dst_i64,
                                               seq * p.dst_seq_stride + t * p.dst_step_stride)
                                  : p.pad_slot_id;
            else
                s.w = (t == len - 1) ? r : p.pad_slot_id;
        } else {
            s.w = p.dst ? load_index(p.dst, p.dst_i64, seq) : r;
        }
        return s;
    };
    auto stage_store = [&](const Stage& s, int buf) {
        if (ht < RB) {
            float xv = 0.f, dA = 0.f, x = 0.f, z = 0.f;
            if (stages_row) {
                x = widen_io<IT>(s.x);
                z = widen_io<IT>(s.z);
                float v = s.dt + bias_h;
                if (p.dt_softplus) v = softplus_f32(v);
                dA = expf(a_h * v);
                xv = v * x;
            }
            row_slot(buf, kXV, ht) = xv;
            row_slot(buf, kDA, ht) = dA;
            row_slot(buf, kX, ht) = x;
            row_slot(buf, kZ, ht) = z;
        }
        if (stages_bc) {
            sB[buf * N + tid] = widen_io<IT>(s.b);
            sC[buf * N + tid] = widen_io<IT>(s.c);
        }
    };

    // Token 0's operands are requested before the state, so waiting for them does
    // not wait for the state.
    Stage stage = stage_load(0);

    // ---- state gather: RL row-loads per lane, all in flight at once. Rows past
    // headdim (a ragged last block) read the last row instead and are never stored.
    const size_t slot_bytes = static_cast<size_t>(H) * P * N * sizeof(ST);
    const size_t head_bytes = static_cast<size_t>(P) * N * sizeof(ST);
    const bool full_block = rb * RB + RB <= P;
    unsigned off[RL];
#pragma unroll
    for (int i = 0; i < RL; ++i) {
        const int pr = rb * RB + wave * (RPI * RL) + i * RPI + rg;
        off[i] = (static_cast<unsigned>(pr < P ? pr : P - 1) * N + n0) * sizeof(ST);
    }
    words_t raw[RL];
    {
        const char* tile = static_cast<const char*>(p.state) + r * slot_bytes + h * head_bytes;
#pragma unroll
        for (int i = 0; i < RL; ++i)
            raw[i] = __builtin_nontemporal_load(reinterpret_cast<const words_t*>(tile + off[i]));
    }

    float s[RL][VEC];
    auto token = [&](int64_t t, bool first) {
        const int buf = static_cast<int>(t & 1);
        stage_store(stage, buf);
        const int64_t w = uniform64(stage.w);
        lds_barrier();
        if constexpr (PACKED) {
            if (t + 1 < len) stage = stage_load(t + 1);
        }
        if (first) {
#pragma unroll
            for (int i = 0; i < RL; ++i)
#pragma unroll
                for (int k = 0; k < W; ++k)
                    Pack<ST>::widen(raw[i][k], &s[i][k * Pack<ST>::kPerWord]);
        }

        float bv[VEC], cv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            bv[e] = sB[buf * N + n0 + e];
            cv[e] = sC[buf * N + n0 + e];
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int pl = wave * (RPI * RL) + i * RPI + rg;
            const float dA = row_slot(buf, kDA, pl);
            const float xv = row_slot(buf, kXV, pl);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s[i][e] = fmaf(s[i][e], dA, xv * bv[e]);
                acc = fmaf(s[i][e], cv[e], acc);
            }
            acc = group_sum<LPR>(acc);
            if ((lane % LPR) == 0) row_slot(buf, kY, pl) = acc;
        }

        // ---- state scatter for this token
        if (!p.disable_state_update && slot_ok(w, p)) {
            char* tile = static_cast<char*>(p.state) + w * slot_bytes + h * head_bytes;
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                words_t o;
#pragma unroll
                for (int k = 0; k < W; ++k) o[k] = Pack<ST>::narrow(&s[i][k * Pack<ST>::kPerWord]);
                const int pr = rb * RB + wave * (RPI * RL) + i * RPI + rg;
                if (full_block || pr < P)
                    __builtin_nontemporal_store(o, reinterpret_cast<words_t*>(tile + off[i]));
            }
        }
        lds_barrier();

        // ---- epilogue: one lane per row
        if (stages_row) {
            float y = row_slot(buf, kY, ht) + d_h * row_slot(buf, kX, ht);
            if (p.z) y *= silu_f32(row_slot(buf, kZ, ht));
            store_io<IT>(p.out, ((begin + t) * H + h) * P + prow, y);
        }
    };

    token(0, true);
    if constexpr (PACKED) {
        for (int64_t t = 1; t < len; ++t) token(t, false);
    }
}

// ---------------------------------------------------------------- launchers

template <typename ST, typename IT, int N>
hipError_t launch_instance(const KernelParams& p, dim3 grid, dim3 block, hipStream_t stream) {
    const size_t lds = sizeof(float) * lds_floats(N, p.heads_per_block);
    if (p.packed)
        hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, true>), grid, block, lds, stream, p);
    else
        hipLaunchKernelGGL((ssu_update_kernel<ST, IT, N, false>), grid, block, lds, stream, p);
    return hipGetLastError();
}

template <typename ST, typename IT>
hipError_t launch_dstate(const KernelParams& p, int dstate, dim3 grid, dim3 block,
                         hipStream_t stream) {
    switch (dstate) {
        case 16: return launch_instance<ST, IT, 16>(p, grid, block, stream);
        case 32: return launch_instance<ST, IT, 32>(p, grid, block, stream);
        case 64: return launch_instance<ST, IT, 64>(p, grid, block, stream);
        case 128: return launch_instance<ST, IT, 128>(p, grid, block, stream);
        case 256: return launch_instance<ST, IT, 256>(p, grid, block, stream);
        default: return hipErrorInvalidValue;
    }
}

// io dtype codes follow ssu_dtype: 0 fp32, 1 fp16, 2 bf16.
template <typename ST>
hipError_t launch_state(const KernelParams& p, int io_dtype, int dstate, dim3 grid, dim3 block,
                        hipStream_t stream) {
    switch (io_dtype) {
        case 0: return launch_dstate<ST, float>(p, dstate, grid, block, stream);
        case 1: return launch_dstate<ST, _Float16>(p, dstate, grid, block, stream);
        case 2: return launch_dstate<ST, __bf16>(p, dstate, grid, block, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssu
