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
                         double *out);

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
    int64_t pad_slot_id, int disable_state_update, double *out);

#ifdef __cplusplus
}
#endif

#endif /* SSU_ORACLE_H */
