/*
 * ssu.h -- C ABI of the Mamba-2 selective state update (SSU) decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * Two entry points, one kernel family:
 *   ssu_one_token      one token per sequence (the plain decode step);
 *   ssu_packed_varlen  packed variable-length rows described by cu_seqlens, one
 *                      destination slot per token, and an acceptance count that
 *                      picks the read slot (the multi-token / MTP decode step).
 * The split follows the call shapes the MATE documentation page "Source code for
 * mate.mamba" routes to its two kernels (module docstring, and the route test at
 * the end of `selective_state_update`); here the caller names the route, so no
 * device-to-host read is ever needed to choose it.
 *
 * The update, per (sequence, head h, row p < headdim), with g = h / (nheads /
 * ngroups) the group of head h (contiguous blocks of heads per group):
 *     v   = dt (+ dt_bias[h]);   v = log(1 + exp(v)) when dt_softplus
 *     dA  = exp(A[h] * v)
 *     s[n] <- s[n] * dA + v * B[g, n] * x[h, p]          for n < dstate
 *     y   = sum_n s[n] * C[g, n]  (+ D[h] * x[h, p])
 *     y  *= z * sigmoid(z)                                when z is given
 * i.e. the Mamba-2 selective state space step (Dao & Gu, ICML 2024) with the
 * block's SiLU output gate; the output uses the updated state. Arithmetic is
 * fp32; the state is read from and written to its storage dtype (stores round to
 * nearest even); out is written in the io dtype.
 *
 * Memory and ownership. Every data pointer is a device pointer owned by the
 * caller; the library keeps none of them after the call returns. A call makes
 * exactly one kernel launch on `stream` (a hipStream_t; NULL is the null stream)
 * or none when there is no work. It allocates nothing, copies nothing between
 * host and device and never synchronises, so it may be recorded into a HIP graph.
 * Layouts are dense row-major:
 *   state  [nslots, nheads, headdim, dstate]   state_dtype, 16-byte aligned
 *   x, z, out  [rows, nheads, headdim]         io_dtype
 *   B, C   [rows, ngroups, dstate]             io_dtype
 *   dt     [rows, nheads] (dt_per_dim = 0) or [rows, nheads, headdim] (= 1), fp32
 *   A, D, dt_bias  [nheads] fp32 (one value per head)
 * For ssu_one_token, rows = batch and row b is sequence b.
 *
 * Slots. A slot id is used only if it differs from pad_slot_id and lies in
 * [0, nslots); otherwise it is inert: an inert read slot makes the whole
 * sequence do nothing (no state read or write, its out rows are not written); an
 * inert destination drops only that state write. The same validity mask guards
 * every load and store of the ReplaySSM tracker kernels on the vLLM page
 * "vllm.model_executor.layers.mamba.ops.ssu_dispatch". Data on the device is
 * never checked on the host: bad slot ids, acceptance counts or row ranges make
 * the affected sequence inert instead of raising.
 *
 * Caller preconditions (not checked; results are unspecified otherwise): no two
 * sequences write the same slot, no sequence writes a slot another sequence
 * reads, cu_seqlens is non-decreasing, and `out` does not overlap any input.
 * A sequence may write the slot it reads (in-place update).
 *
 * Stochastic rounding. With a 16-bit state and rand_seed set, every stored state
 * element is rounded stochastically instead of to nearest: with q the spacing of
 * the state format at |v|, m = floor(|v| / q) and frac = |v| / q - m, the stored
 * magnitude is (m + 1) q when U >= 1 - frac and m q otherwise (infinite past the
 * largest finite value), U being a uniform number of 16 (bf16) or 24 (fp16)
 * random bits divided by 2^16 or 2^24. The bits come from Philox4x32 (Salmon et
 * al., SC'11) with philox_rounds rounds, key (seed mod 2^32, seed / 2^32) and a
 * counter per group of elements. Element e = (h * headdim + p) * dstate + n of
 * the state written by packed row r (row b for ssu_one_token) takes:
 *   fp16: counter (e / 4, r mod 2^32, r / 2^32, 0); word w = e % 4 of the
 *         output; the top 24 bits of that word;
 *   bf16: counter (e / 8, r mod 2^32, r / 2^32, 0); word w = (e % 8) / 2 of the
 *         output; its low 16 bits for even e, its high 16 bits for odd e.
 * (Words are numbered 0..3 in the order Philox returns them.) The vLLM
 * dispatch page forwards exactly these two knobs (a device seed and a round count,
 * 10 by default) when stochastic rounding is enabled; the rule and the counter
 * layout are this library's. `out` is always rounded to nearest.
 *
 * Errors. Each entry point returns an ssu_status. On failure nothing is launched
 * and ssu_last_error() names the offending argument or capability. Calls from
 * different host threads are independent; the error text is per thread.
 */
#ifndef SSU_H
#define SSU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSU_ABI_VERSION 1

typedef enum ssu_dtype {
    SSU_F32 = 0,
    SSU_F16 = 1,
    SSU_BF16 = 2
} ssu_dtype;

typedef enum ssu_index_dtype {
    SSU_I32 = 0,
    SSU_I64 = 1
} ssu_index_dtype;

typedef enum ssu_status {
    SSU_OK = 0,
    SSU_ERR_INVALID_ARGUMENT = 1, /* inconsistent sizes, null required pointer, ... */
    SSU_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement */
    SSU_ERR_LAUNCH = 3            /* the HIP runtime refused the launch */
} ssu_status;

/*
 * Operands common to both entry points. Operand roles and dtypes follow the
 * module docstring and the shape checks of `selective_state_update` on the MATE
 * page "Source code for mate.mamba"; fp32 io is accepted as well.
 */
typedef struct ssu_operands {
    void *state;              /* [nslots, nheads, headdim, dstate], read and written */
    int32_t state_dtype;      /* ssu_dtype */
    int64_t nslots;           /* >= 1 */
    int64_t nheads;           /* >= 1, multiple of ngroups */
    int64_t headdim;          /* >= 1 */
    int64_t dstate;           /* 16, 32, 64, 128 or 256 */
    int64_t ngroups;          /* >= 1 */

    const void *x;            /* [rows, nheads, headdim], required */
    const void *B;            /* [rows, ngroups, dstate], required */
    const void *C;            /* [rows, ngroups, dstate], required */
    const void *z;            /* [rows, nheads, headdim] or NULL (no gate) */
    void *out;                /* [rows, nheads, headdim], required, written */
    int32_t io_dtype;         /* ssu_dtype of x, B, C, z and out */

    const float *dt;          /* fp32, see dt_per_dim, required */
    int32_t dt_per_dim;       /* 0: dt is [rows, nheads]; 1: [rows, nheads, headdim] */
    const float *A;           /* [nheads], required */
    const float *D;           /* [nheads] or NULL (no skip term) */
    const float *dt_bias;     /* [nheads] or NULL (no bias) */
    int32_t dt_softplus;      /* nonzero: v = softplus(dt + dt_bias) */

    int64_t pad_slot_id;      /* slot id meaning "no slot"; -1 by convention */
    int32_t disable_state_update; /* nonzero: compute out, write no state */
    const void *rand_seed;    /* device pointer to one int64 seed, or NULL: with a
                                 16-bit state, stored states are rounded
                                 stochastically (no effect on an fp32 state) */
    int32_t philox_rounds;    /* Philox rounds for rand_seed; 0 means 10 */

    int32_t heads_per_block;  /* launch shape: heads of one group per workgroup,
                                 0 = library default, else 1, 2 or 4 dividing
                                 nheads / ngroups (at most 2 for dstate 256
                                 and for ssu_packed_varlen) */
    int32_t loads_per_lane;   /* launch shape: 16-byte state loads each lane keeps in
                                 flight, 0 = library default, else 2 or 4 (a lane
                                 keeps fewer where dstate rows are too short to
                                 give it that many) */
    int32_t tile_order;       /* launch shape: 0 = library default, 1 = each XCD takes
                                 a contiguous range of tiles, 2 = hardware order, 3 = each
                                 XCD takes an equal contiguous share (a block of heads) of
                                 every sequence's tiles (as 1 when a sequence's tiles do
                                 not split evenly over the 8 XCDs) */
} ssu_operands;

/*
 * ssu_one_token: one decode token per sequence.
 * Slot vectors: src_slots[b] is the slot sequence b reads (NULL: slot b);
 * dst_slots[b] the slot it writes (NULL: the slot it read). MATE page,
 * `_slot_vector` (a missing vector is the identity).
 */
typedef struct ssu_one_token_args {
    uint32_t struct_size;     /* sizeof(ssu_one_token_args) */
    ssu_operands op;
    int64_t batch;            /* sequences = rows, >= 0; 0 launches nothing */
    const void *src_slots;    /* [batch] or NULL */
    int32_t src_dtype;        /* ssu_index_dtype of src_slots */
    const void *dst_slots;    /* [batch] or NULL */
    int32_t dst_dtype;        /* ssu_index_dtype of dst_slots */
} ssu_one_token_args;

/*
 * ssu_packed_varlen: packed variable-length multi-token decode.
 * Sequence b owns rows [cu_seqlens[b], cu_seqlens[b+1]); an empty range does
 * nothing, a range outside [0, rows] or running backwards is inert. With
 * cu_seqlens NULL and seq_len > 0 the sequences are regular: sequence b owns rows
 * [b * seq_len, (b + 1) * seq_len) and rows must equal nseq * seq_len -- the dense
 * [batch, steps, heads, dim] layout, which the MATE page runs as packed varlen
 * with regular starts (`selective_state_update`, `_dense_seq_starts`). The state
 * chains from token to token of a sequence in fp32 registers, without rounding to
 * the storage dtype in between.
 *   read slot   k = num_accepted[b] (NULL: 1); the slot is
 *               src_table[b * src_seq_stride + (k - 1) * src_step_stride];
 *               k outside [1, steps] makes the sequence inert. A NULL src_table
 *               means sequence b reads slot b (then num_accepted must be NULL).
 *   write slots token t writes dst_table[b * dst_seq_stride + t * dst_step_stride]
 *               for t < steps (positions t >= steps are inert). A NULL dst_table
 *               writes the state after the last token back to the read slot.
 * Tables follow the MATE page "Source code for mate.mamba": `_slot_table`
 * (entry = sequence * seq_stride + position * step_stride; a contiguous
 * [nseq, steps] table has strides (steps, 1), a flat per-row table (1, 1)) and
 * `_packed_selective_state_update` (the acceptance count picks the read entry and
 * needs a read table; cu_seqlens and num_accepted share one dtype).
 * The tables must hold every entry these formulas reach for k <= steps, t < steps.
 */
typedef struct ssu_packed_args {
    uint32_t struct_size;     /* sizeof(ssu_packed_args) */
    ssu_operands op;
    int64_t rows;             /* packed rows (= cu_seqlens[nseq] for valid data), >= 0 */
    int64_t nseq;             /* sequences, >= 0; 0 launches nothing */
    const void *cu_seqlens;   /* [nseq + 1]; or NULL with seq_len > 0 */
    int64_t seq_len;          /* rows per sequence when cu_seqlens is NULL, else 0 */
    const void *num_accepted; /* [nseq] or NULL */
    int32_t meta_dtype;       /* ssu_index_dtype of cu_seqlens and num_accepted */
    const void *src_table;    /* or NULL */
    int32_t src_dtype;        /* ssu_index_dtype */
    int64_t src_seq_stride, src_step_stride; /* >= 0, in entries */
    const void *dst_table;    /* or NULL */
    int32_t dst_dtype;        /* ssu_index_dtype */
    int64_t dst_seq_stride, dst_step_stride; /* >= 0, in entries */
    int64_t steps;            /* table width; >= 1 when a table is given */
} ssu_packed_args;

/*
 * ReplaySSM ring trackers: three per-slot counters kept beside the state cache
 * when decode replays a ring of cached inputs from a checkpointed state
 * (ring_start, prev_num_accepted, prev_query_len). The update and the delayed
 * commit follow the two tracker kernels of the vLLM `ssu_dispatch` module source
 * (`update_replayssm_ring_trackers`, `commit_replayssm_ring_trackers`).
 *
 * Position i < n names slot slots[i * slot_stride] (a 2-D [n, w] slot table is
 * passed with slot_stride w: its first column). Positions whose slot is pad or
 * outside [0, num_states) are skipped. Per named slot:
 *   ssu_ring_update, reset != 0: all three counters become 0;
 *   ssu_ring_update, reset == 0: one token decoded -- when prev_num_accepted + 1
 *     exceeds logical_window, ring_start advances by prev_num_accepted (mod
 *     ring_buffer_len) and prev_num_accepted becomes 1, else it grows by 1;
 *   ssu_ring_commit: settles the previous speculative window. With
 *     prev_query_len 0 (none), prev_num_accepted becomes 0. Otherwise, when
 *     prev_num_accepted + prev_query_len exceeds logical_window, ring_start
 *     advances by prev_num_accepted (mod ring_buffer_len) and prev_num_accepted
 *     becomes num_accepted[i]; else num_accepted[i] is added to it. Then
 *     prev_query_len = query_start_loc[i + 1] - query_start_loc[i].
 * Slots named at valid positions must be distinct. One launch, no allocation,
 * no synchronisation; n == 0 launches nothing.
 */
typedef struct ssu_ring_args {
    uint32_t struct_size;          /* sizeof(ssu_ring_args) */
    void *ring_start;              /* [num_states] */
    void *prev_num_accepted;       /* [num_states] */
    void *prev_query_len;          /* [num_states] */
    int32_t tracker_dtype;         /* ssu_index_dtype of the three counters */
    int64_t num_states;            /* >= 0 */
    const void *slots;             /* n entries, slot_stride apart */
    int32_t slot_dtype;            /* ssu_index_dtype */
    int64_t slot_stride;           /* >= 0, in entries */
    int64_t n;                     /* positions, >= 0 */
    const void *num_accepted;      /* commit: [n] */
    const void *query_start_loc;   /* commit: [n + 1] */
    int32_t meta_dtype;            /* commit: ssu_index_dtype of the two above */
    int32_t reset;                 /* update: nonzero resets */
    int64_t logical_window;        /* >= 0 (advance, commit) */
    int64_t ring_buffer_len;       /* >= 1 (advance, commit) */
    int64_t pad_slot_id;
} ssu_ring_args;

/* Reset or advance the trackers of the named slots. Returns an ssu_status. */
int ssu_ring_update(const ssu_ring_args *args, void *stream);

/* Commit the previous speculative window of the named slots. Returns an ssu_status. */
int ssu_ring_commit(const ssu_ring_args *args, void *stream);

/* Run the one-token update on `stream`. Returns an ssu_status. */
int ssu_one_token(const ssu_one_token_args *args, void *stream);

/* Run the packed variable-length update on `stream`. Returns an ssu_status. */
int ssu_packed_varlen(const ssu_packed_args *args, void *stream);

/* Text of the last failure on this host thread ("" after a success). */
const char *ssu_last_error(void);

/* SSU_ABI_VERSION of the loaded library. */
int ssu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSU_H */
