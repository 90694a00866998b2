/*
 * ssu_oracle.h -- plain fp64 CPU reference of the Mamba-2 selective state update.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code, header or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * Every floating-point operand is an fp64 array; every index operand is int64.
 * Callers widen fp16/bf16/fp32 data to fp64 first (exact for all three formats).
 * The state cache is read from `state_in` and the result is written to
 * `state_out` (a separate buffer of the same shape): the call first copies
 * `state_in` into `state_out`, then overwrites the destination slots, so every
 * read sees the state as it was before the call.
 *
 * Shapes (row-major, contiguous):
 *   state_in / state_out  [nslots, nheads, headdim, dstate]
 *   x, z, out             [rows, nheads, headdim]
 *   dt                    [rows, nheads]            (dt_per_dim == 0)
 *                         [rows, nheads, headdim]   (dt_per_dim != 0)
 *   A, D, dt_bias         [nheads]
 *   B, C                  [rows, ngroups, dstate]
 *
 * Return value: 0 on success, -1 if an argument is inconsistent (null required
 * pointer, non-positive size, nheads not a multiple of ngroups, state_in equal
 * to state_out). Data-dependent conditions (pad or out-of-range slots, bad
 * acceptance counts, bad row ranges) are not errors: they make the affected
 * sequence or write inert, as documented per function.
 */
#ifndef SSU_ORACLE_H
#define SSU_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Stochastic rounding of stored states. With sr_format != 0 every state the call
 * writes is rounded stochastically to fp16 (sr_format 1) or bf16 (2) -- the
 * fp64 result holds the exact 16-bit value -- using Philox4x32 with
 * philox_rounds rounds keyed by the 64-bit rand_seed. Element
 * e = (h * headdim + p) * dstate + n of the state written by packed row `row`
 * draws its random bits from Philox(counter = (e / G, row % 2^32, row / 2^32, 0)):
 *   fp16 (G = 4): the top 24 bits of word e % 4;
 *   bf16 (G = 8): 16 bits of word (e % 8) / 2, its low half for even e and its
 *                 high half for odd e.
 * With sr_format 0 stored states are the unrounded fp64 values.
 * row_base: the number, in the call the random bits are counted over, of this
 * problem's row 0 -- 0 for a whole call; for a problem cut out of a larger call
 * (a run of consecutive sequences), the packed row where the cut begins, so the
 * counters keep their call-wide row numbers.
 */
typedef struct {
    int sr_format;          /* 0 none, 1 fp16, 2 bf16 */
    uint64_t rand_seed;
    int philox_rounds;
    int64_t row_base;
} oracle_rounding;

/* One token per sequence (row b is sequence b). src/dst may be NULL. */
int oracle_ssu_one_token(const double *state_in, double *state_out,
                         int64_t nslots, int64_t nheads, int64_t headdim,
                         int64_t dstate, int64_t ngroups, int64_t batch,
                         const double *x, const double *dt, int dt_per_dim,
                         const double *A, const double *B, const double *C,
                         const double *D, const double *z,
                         const double *dt_bias, int dt_softplus,
                         const int64_t *src, const int64_t *dst,
                         int64_t pad_slot_id, int disable_state_update,
                         const oracle_rounding *rounding, double *out);

/* Packed variable-length form: sequence b owns rows [cu[b], cu[b+1]). */
int oracle_ssu_packed_varlen(
    const double *state_in, double *state_out, int64_t nslots, int64_t nheads,
    int64_t headdim, int64_t dstate, int64_t ngroups, int64_t rows,
    int64_t nseq, const int64_t *cu_seqlens, const int64_t *num_accepted,
    const int64_t *src_table, int64_t src_seq_stride, int64_t src_step_stride,
    const int64_t *dst_table, int64_t dst_seq_stride, int64_t dst_step_stride,
    int64_t steps, const double *x, const double *dt, int dt_per_dim,
    const double *A, const double *B, const double *C, const double *D,
    const double *z, const double *dt_bias, int dt_softplus,
    int64_t pad_slot_id, int disable_state_update, const oracle_rounding *rounding,
    double *out);

/* Philox4x32 (Salmon et al., SC'11): `rounds` rounds of the 4x32 round function
 * on counter[4] with key[2], the key bumped by the Weyl constants between
 * rounds. Writes the four output words to out[4]. */
void oracle_philox4x32(const uint32_t counter[4], const uint32_t key[2], int rounds,
                       uint32_t out[4]);

/* Stochastic rounding of v to fp16 (format 1) or bf16 (2) with random word w,
 * for n values: out[i] = SR(v[i], w[i]). */
void oracle_round_stochastic(const double *v, const uint32_t *w, int64_t n, int format,
                             double *out);

/*
 * ReplaySSM ring trackers: three per-slot counters (ring_start,
 * prev_num_accepted, prev_query_len), int64 here, [num_states] each. Position i
 * < n names slot slots[i * slot_stride]; an invalid slot (pad or outside
 * [0, num_states)) is skipped. Slots of valid positions are assumed distinct.
 *
 * ring_update with reset != 0 zeroes the three counters of every named slot;
 * otherwise it advances each named slot's ring by one decoded token.
 * ring_commit advances each named slot by the accepted prefix of the previous
 * speculative window (num_accepted[i]) and records the current window's length
 * (query_start_loc[i + 1] - query_start_loc[i]).
 * Return value: 0, or -1 for inconsistent arguments (negative sizes, a ring of
 * fewer than one entry, a null array that is needed).
 */
int oracle_ring_update(int64_t *ring_start, int64_t *prev_num_accepted,
                       int64_t *prev_query_len, int64_t num_states,
                       const int64_t *slots, int64_t slot_stride, int64_t n,
                       int reset, int64_t logical_window,
                       int64_t ring_buffer_len, int64_t pad_slot_id);

int oracle_ring_commit(int64_t *ring_start, int64_t *prev_num_accepted,
                       int64_t *prev_query_len, int64_t num_states,
                       const int64_t *slots, int64_t slot_stride, int64_t n,
                       const int64_t *num_accepted, const int64_t *query_start_loc,
                       int64_t logical_window, int64_t ring_buffer_len,
                       int64_t pad_slot_id);

/*
 * SSD chunked prefill over packed variable-length sequences.
 *   x, z, out [tokens, nheads, headdim]; dt [tokens, nheads];
 *   B, C [tokens, ngroups, dstate]; A, dt_bias [nheads];
 *   D [nheads] (D_per_dim == 0) or [nheads, headdim] (D_per_dim != 0), or NULL;
 *   initial_states, final_states [batch, nheads, headdim, dstate] (either NULL);
 *   chunk_states [nchunks, nheads, headdim, dstate].
 * Chunk c covers tokens [cu_chunk_seqlens[c], cu_chunk_seqlens[c+1]) (at most
 * chunk_size of them) and belongs to request seq_idx[c]. A chunk opens a
 * sequence when c == 0 or seq_idx[c] != seq_idx[c-1]; it then enters with
 * initial_states[seq_idx[c]] (zeros if NULL), otherwise with the state the
 * previous chunk left. Inside a chunk the recurrence runs token by token with
 * v = clamp(softplus?(dt + dt_bias), dt_min, dt_max). chunk_states[c] is the
 * state after chunk c; final_states[b] = chunk_states[last_chunk_indices[b]].
 * Rows of `out` no chunk covers are left as they are.
 * Returns -1 for inconsistent arguments, including chunk ranges outside
 * [0, tokens], running backwards or longer than chunk_size, a seq_idx outside
 * [0, batch) when initial states are given, and last_chunk_indices outside
 * [0, nchunks).
 */
int oracle_ssd_prefill(int64_t tokens, int64_t nheads, int64_t headdim, int64_t dstate,
                       int64_t ngroups, const double *x, const double *dt, const double *A,
                       const double *B, const double *C, const double *D, int D_per_dim,
                       const double *z, const double *dt_bias, int dt_softplus,
                       double dt_min, double dt_max, int64_t chunk_size, int64_t nchunks,
                       const int64_t *cu_chunk_seqlens, const int64_t *seq_idx, int64_t batch,
                       const int64_t *last_chunk_indices, const double *initial_states,
                       double *out, double *chunk_states, double *final_states);

#ifdef __cplusplus
}
#endif

#endif /* SSU_ORACLE_H */
