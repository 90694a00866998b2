/*
 * ssu_oracle.c -- plain fp64 CPU reference of the Mamba-2 selective state update.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library; the GPU library never calls it and
 * the two share no code. Loops run in the plain order sequence -> head -> row ->
 * dstate, in fp64, with no blocking or reordering.
 *
 * What is computed, and where it comes from:
 *
 *  - The recurrence. The pages name the operands and their roles but do not write
 *    the update; it is the Mamba-2 selective state space step (Dao & Gu,
 *    "Transformers are SSMs", ICML 2024, the SSD recurrence
 *    h_t = exp(dt_t * A) h_{t-1} + dt_t B_t x_t,  y_t = C_t . h_t + D x_t), with
 *    the Mamba-2 block's output gate y * silu(z). Per (sequence, head h, row p):
 *        v   = dt[h] (+ dt_bias[h]);  v = softplus(v) when requested
 *        dA  = exp(A[h] * v)
 *        s'  = s * dA + v * B[g, n] * x[h, p]            for every n < dstate
 *        y   = sum_n s'[n] * C[g, n]  (+ D[h] * x[h, p])
 *        y  *= z * sigmoid(z)                            when z is given
 *    The output uses the post-update state; D enters before the gate; the bias is
 *    added before the softplus and no clamp is applied.
 *  - Operand roles, dtypes and per-head A/D/dt_bias: MATE docs, "Source code for
 *    mate.mamba", module docstring (supported configuration) and the shape checks
 *    of `selective_state_update`.
 *  - Head-to-group map: heads form contiguous blocks of nheads/ngroups per group
 *    (same page, the `head_ratio = heads // groups` specialisation key of the
 *    prewarm entry, and the heads-divisible-by-groups check of the SSD entry).
 *  - Slot vectors default to the identity (same page, `_slot_vector`); a missing
 *    destination means the update is written back where it was read.
 *  - Slot validity: a slot is used only when it differs from pad_slot_id and lies
 *    in [0, nslots) -- the same mask the ring-tracker kernels of the vLLM
 *    `ssu_dispatch` module apply before every load and store. An invalid read slot
 *    makes the whole sequence inert (no state read or write, its `out` rows are
 *    left as they are); an invalid destination only drops that state write.
 *  - Packed form: MATE docs, `mate.mamba`, module docstring and
 *    `_packed_selective_state_update`: rows are grouped by cu_seqlens, the
 *    acceptance count picks the entry of the read table (entry k-1), each token
 *    has its own destination entry, and the state chains token to token inside a
 *    sequence without rounding in between.
 *  - Table addressing: `_slot_table` docstring: entry = sequence * seq_stride +
 *    position * step_stride.
 *  - The dense [batch, steps, ...] form is the packed form with regular starts
 *    (`selective_state_update` body), so it needs no function of its own here.
 *  - Stochastic rounding of 16-bit state: the vLLM dispatch page forwards a
 *    random seed and a Philox round count (default 10) to the state update when
 *    stochastic rounding is enabled; the rounding rule and the random-number
 *    layout are not on the pages. Reading taken here: unbiased stochastic
 *    rounding of the exact state value to the target format (round away from
 *    zero with probability equal to the fraction of the quantum the value passes),
 *    driven by Philox4x32 as published (Salmon, Moraes, Dror, Shaw, "Parallel
 *    random numbers: as easy as 1, 2, 3", SC'11), with the counter layout
 *    documented in ssu_oracle.h.
 *  - ReplaySSM ring trackers: the update / reset and the delayed commit of the
 *    vLLM `ssu_dispatch` module source (the two tracker kernels and their
 *    wrappers `update_replayssm_ring_trackers` and
 *    `commit_replayssm_ring_trackers`), restated per slot below.
 *  - SSD chunked prefill: the contract of `ssd_combined_fwd_varlen` on the MATE
 *    page (its docstring and argument checks). The chunked algorithm computes,
 *    up to rounding order, the same recurrence run token by token over each
 *    sequence (the structured-state-space duality of the SSD paper, sections 5
 *    and 6), so the oracle is that plain recurrence with the contract's chunk
 *    bookkeeping: which tokens a chunk covers, where its entering state comes
 *    from, and which states are returned.
 */
#include "ssu_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* softplus(v) = log(1 + exp(v)), written so that neither branch overflows. */
static double softplus(double v) {
    if (v > 0.0) return v + log1p(exp(-v));
    return log1p(exp(v));
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static int slot_valid(int64_t slot, int64_t pad_slot_id, int64_t nslots) {
    return slot != pad_slot_id && slot >= 0 && slot < nslots;
}

typedef struct {
    int64_t nslots, nheads, headdim, dstate, ngroups;
    const double *x, *dt, *A, *B, *C, *D, *z, *dt_bias;
    int dt_per_dim, dt_softplus;
} problem;

/* ------------------------------------------------------ stochastic rounding */

/* One Philox4x32 round: two 32x32->64 products of counter words 0 and 2 with
 * the multipliers; the high halves are mixed with the other two counter words
 * and the key, the low halves pass through. */
void oracle_philox4x32(const uint32_t counter[4], const uint32_t key[2], int rounds,
                       uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;   /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;   /* key increments */
    uint32_t c0 = counter[0], c1 = counter[1], c2 = counter[2], c3 = counter[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < rounds; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t p0 = (uint64_t)M0 * c0;
        const uint64_t p1 = (uint64_t)M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* SR(v): q is the target format's spacing at |v| (2^(e - mantissa bits), with e
 * clamped to the smallest normal exponent so subnormals share one spacing),
 * m = floor(|v| / q), frac = |v| / q - m. The result is m q, or (m + 1) q when
 * the k-bit uniform U taken from the top of w satisfies U >= 1 - frac; past the
 * largest finite value it is infinite. NaN, infinities and zeros pass through. */
static double round_stochastic(double v, uint32_t w, int format) {
    if (v != v || v == 0.0 || isinf(v)) return v;
    const int mant = format == 1 ? 10 : 7;           /* explicit mantissa bits */
    const int emin = format == 1 ? -14 : -126;       /* smallest normal exponent */
    const int kbits = format == 1 ? 24 : 16;         /* random bits used */
    const double maxfin = format == 1 ? 65504.0 : ldexp(2.0 - ldexp(1.0, -7), 127);
    const double a = fabs(v);
    int e;
    frexp(a, &e);                                    /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                                          /* a in [2^e, 2^(e+1)) */
    const int qexp = (e > emin ? e : emin) - mant;
    const double t = ldexp(a, -qexp);
    const double m = floor(t);
    const double frac = t - m;
    const double U = ldexp((double)(w >> (32 - kbits)), -kbits);
    /* U >= 1 - frac, decided exactly: U - 1 is exact and a rounded sum keeps
     * the sign of the exact one. */
    double r = ldexp(m + ((U - 1.0) + frac >= 0.0 ? 1.0 : 0.0), qexp);
    if (r > maxfin) r = INFINITY;
    return v < 0 ? -r : r;
}

void oracle_round_stochastic(const double *v, const uint32_t *w, int64_t n, int format,
                             double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_stochastic(v[i], w[i], format);
}

/* Round the fp64 state s ([nheads, headdim, dstate]) written by packed row `row`
 * into dst, stochastically when requested. */
static void store_state(double *dst, const double *s, int64_t elems, int64_t row,
                        const oracle_rounding *rd) {
    if (!rd || rd->sr_format == 0) {
        memcpy(dst, s, (size_t)elems * sizeof(double));
        return;
    }
    const uint32_t key[2] = {(uint32_t)rd->rand_seed, (uint32_t)(rd->rand_seed >> 32)};
    const int bf16 = rd->sr_format == 2;
    row += rd->row_base;                         /* the call-wide row number */
    const int64_t group = bf16 ? 8 : 4;          /* elements per Philox call */
    for (int64_t e = 0; e < elems; ++e) {
        const uint32_t ctr[4] = {(uint32_t)(e / group), (uint32_t)row,
                                 (uint32_t)((uint64_t)row >> 32), 0};
        uint32_t words[4];
        oracle_philox4x32(ctr, key, rd->philox_rounds, words);
        uint32_t w;
        if (bf16) {
            const uint32_t word = words[(e % 8) / 2];
            const uint32_t bits16 = (e % 2) ? (word >> 16) : (word & 0xFFFFu);
            w = bits16 << 16;                    /* round_stochastic reads the top bits */
        } else {
            w = words[e % 4];
        }
        dst[e] = round_stochastic(s[e], w, rd->sr_format);
    }
}

/*
 * Advance one sequence's fp64 state `s` ([nheads, headdim, dstate]) by the token
 * in packed row `row`, and write that row of `out`.
 */
static void step_token(const problem *pb, double *s, int64_t row, double *out) {
    const int64_t H = pb->nheads, P = pb->headdim, N = pb->dstate;
    const int64_t heads_per_group = H / pb->ngroups;
    for (int64_t h = 0; h < H; ++h) {
        const int64_t g = h / heads_per_group;
        const double *Bg = pb->B + (row * pb->ngroups + g) * N;
        const double *Cg = pb->C + (row * pb->ngroups + g) * N;
        for (int64_t p = 0; p < P; ++p) {
            const int64_t xi = (row * H + h) * P + p;
            double v = pb->dt_per_dim ? pb->dt[xi] : pb->dt[row * H + h];
            if (pb->dt_bias) v += pb->dt_bias[h];
            if (pb->dt_softplus) v = softplus(v);
            const double dA = exp(pb->A[h] * v);
            const double xs = pb->x[xi];
            double *sp = s + (h * P + p) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                sp[n] = sp[n] * dA + v * Bg[n] * xs;
                acc += sp[n] * Cg[n];
            }
            double y = acc;
            if (pb->D) y += pb->D[h] * xs;
            if (pb->z) {
                const double zz = pb->z[xi];
                y *= zz * sigmoid(zz);
            }
            out[xi] = y;
        }
    }
}

static int check_dims(const double *state_in, const double *state_out,
                      const problem *pb) {
    if (!state_in || !state_out || state_in == state_out) return -1;
    if (pb->nslots <= 0 || pb->nheads <= 0 || pb->headdim <= 0 ||
        pb->dstate <= 0 || pb->ngroups <= 0)
        return -1;
    if (pb->nheads % pb->ngroups != 0) return -1;
    return 0;
}

int oracle_ssu_one_token(const double *state_in, double *state_out,
                         int64_t nslots, int64_t nheads, int64_t headdim,
                         int64_t dstate, int64_t ngroups, int64_t batch,
                         const double *x, const double *dt, int dt_per_dim,
                         const double *A, const double *B, const double *C,
                         const double *D, const double *z,
                         const double *dt_bias, int dt_softplus,
                         const int64_t *src, const int64_t *dst,
                         int64_t pad_slot_id, int disable_state_update,
                         const oracle_rounding *rounding, double *out) {
    const problem pb = {nslots, nheads, headdim, dstate, ngroups,
                        x,      dt,     A,       B,      C,
                        D,      z,      dt_bias, dt_per_dim, dt_softplus};
    if (check_dims(state_in, state_out, &pb) != 0 || batch < 0) return -1;
    if (batch > 0 && (!x || !dt || !A || !B || !C || !out)) return -1;

    const int64_t slot_elems = nheads * headdim * dstate;
    memcpy(state_out, state_in, (size_t)(nslots * slot_elems) * sizeof(double));
    double *s = (double *)malloc((size_t)slot_elems * sizeof(double));
    if (!s) return -1;

    for (int64_t b = 0; b < batch; ++b) {
        const int64_t r = src ? src[b] : b;
        const int64_t w = dst ? dst[b] : r;
        if (!slot_valid(r, pad_slot_id, nslots)) continue;
        memcpy(s, state_in + r * slot_elems, (size_t)slot_elems * sizeof(double));
        step_token(&pb, s, b, out);
        if (!disable_state_update && slot_valid(w, pad_slot_id, nslots))
            store_state(state_out + w * slot_elems, s, slot_elems, b, rounding);
    }
    free(s);
    return 0;
}

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
    double *out) {
    const problem pb = {nslots, nheads, headdim, dstate, ngroups,
                        x,      dt,     A,       B,      C,
                        D,      z,      dt_bias, dt_per_dim, dt_softplus};
    if (check_dims(state_in, state_out, &pb) != 0 || rows < 0 || nseq < 0)
        return -1;
    if (nseq > 0 && !cu_seqlens) return -1;
    if (rows > 0 && (!x || !dt || !A || !B || !C || !out)) return -1;
    /* An acceptance count indexes the read table, so it needs one. */
    if (num_accepted && !src_table) return -1;
    if ((src_table || dst_table) && steps <= 0) return -1;

    const int64_t slot_elems = nheads * headdim * dstate;
    memcpy(state_out, state_in, (size_t)(nslots * slot_elems) * sizeof(double));
    double *s = (double *)malloc((size_t)slot_elems * sizeof(double));
    if (!s) return -1;

    for (int64_t b = 0; b < nseq; ++b) {
        const int64_t begin = cu_seqlens[b], end = cu_seqlens[b + 1];
        /* A row range outside [0, rows] or running backwards makes the sequence
         * inert; an empty one has nothing to do. */
        if (begin < 0 || end > rows || end <= begin) continue;

        /* The read slot: entry k-1 of the sequence's read-table row. */
        const int64_t k = num_accepted ? num_accepted[b] : 1;
        int64_t r;
        if (src_table) {
            if (k < 1 || k > steps) continue;
            r = src_table[b * src_seq_stride + (k - 1) * src_step_stride];
        } else {
            r = b;
        }
        if (!slot_valid(r, pad_slot_id, nslots)) continue;

        memcpy(s, state_in + r * slot_elems, (size_t)slot_elems * sizeof(double));
        for (int64_t t = 0; t < end - begin; ++t) {
            step_token(&pb, s, begin + t, out);
            if (disable_state_update) continue;
            int64_t w;
            if (dst_table)
                w = t < steps ? dst_table[b * dst_seq_stride + t * dst_step_stride]
                              : pad_slot_id;
            else
                w = r;
            if (slot_valid(w, pad_slot_id, nslots))
                store_state(state_out + w * slot_elems, s, slot_elems, begin + t, rounding);
        }
    }
    free(s);
    return 0;
}

/*
 * ReplaySSM ring trackers. Per named slot s:
 *  reset:   ring_start = prev_num_accepted = prev_query_len = 0.
 *  advance: one more token was decoded since the checkpoint. If that makes the
 *           count exceed the logical window, the ring start moves past the
 *           tokens counted so far (mod the ring length) and the count restarts
 *           at 1; otherwise the count grows by one. prev_query_len is left alone.
 *  commit:  the previous speculative window (prev_query_len tokens, 0 = none)
 *           is settled with the count accepted from it. When a window exists and
 *           the tokens counted since the checkpoint plus that window would exceed
 *           the logical window, the ring start moves past the counted tokens and
 *           the count becomes the accepted number; otherwise the accepted number
 *           is added to the count. With no window the count becomes 0. Then the
 *           current window's length is recorded.
 */
static int ring_args_ok(const int64_t *a, const int64_t *b, const int64_t *c,
                        int64_t num_states, const int64_t *slots, int64_t n) {
    if (n < 0 || num_states < 0) return 0;
    if (n > 0 && (!slots || !a || !b || !c)) return 0;
    return 1;
}

int oracle_ring_update(int64_t *ring_start, int64_t *prev_num_accepted,
                       int64_t *prev_query_len, int64_t num_states,
                       const int64_t *slots, int64_t slot_stride, int64_t n,
                       int reset, int64_t logical_window,
                       int64_t ring_buffer_len, int64_t pad_slot_id) {
    if (!ring_args_ok(ring_start, prev_num_accepted, prev_query_len, num_states, slots, n))
        return -1;
    if (!reset && ring_buffer_len < 1) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t s = slots[i * slot_stride];
        if (!slot_valid(s, pad_slot_id, num_states)) continue;
        if (reset) {
            ring_start[s] = 0;
            prev_num_accepted[s] = 0;
            prev_query_len[s] = 0;
            continue;
        }
        const int64_t counted = prev_num_accepted[s];
        if (counted + 1 > logical_window) {
            ring_start[s] = (ring_start[s] + counted) % ring_buffer_len;
            prev_num_accepted[s] = 1;
        } else {
            prev_num_accepted[s] = counted + 1;
        }
    }
    return 0;
}

int oracle_ring_commit(int64_t *ring_start, int64_t *prev_num_accepted,
                       int64_t *prev_query_len, int64_t num_states,
                       const int64_t *slots, int64_t slot_stride, int64_t n,
                       const int64_t *num_accepted, const int64_t *query_start_loc,
                       int64_t logical_window, int64_t ring_buffer_len,
                       int64_t pad_slot_id) {
    if (!ring_args_ok(ring_start, prev_num_accepted, prev_query_len, num_states, slots, n))
        return -1;
    if (ring_buffer_len < 1 || (n > 0 && (!num_accepted || !query_start_loc))) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t s = slots[i * slot_stride];
        if (!slot_valid(s, pad_slot_id, num_states)) continue;
        const int64_t counted = prev_num_accepted[s];
        const int64_t window = prev_query_len[s];
        const int64_t accepted = num_accepted[i];
        if (window == 0) {
            prev_num_accepted[s] = 0;
        } else if (counted + window > logical_window) {
            ring_start[s] = (ring_start[s] + counted) % ring_buffer_len;
            prev_num_accepted[s] = accepted;
        } else {
            prev_num_accepted[s] = counted + accepted;
        }
        prev_query_len[s] = query_start_loc[i + 1] - query_start_loc[i];
    }
    return 0;
}

/*
 * SSD chunked prefill. Chunk c covers tokens [cu_chunk_seqlens[c],
 * cu_chunk_seqlens[c+1]). It opens a sequence when c == 0 or seq_idx[c] differs
 * from seq_idx[c-1]; an opening chunk enters with initial_states[seq_idx[c]]
 * (zeros without initial states), any other chunk with the state the previous
 * chunk left. Inside a chunk the tokens run in order through the recurrence:
 *     v  = dt[t, h] (+ dt_bias[h]);  v = softplus(v) when requested;
 *     v  = min(max(v, dt_min), dt_max)
 *     s  = s * exp(A[h] v) + v B[t, g] x[t, h, p]
 *     y  = C[t, g] . s + D x[t, h, p];  y *= z sigmoid(z) when z is given
 * chunk_states[c] is the state after the chunk's last token and
 * final_states[b] = chunk_states[last_chunk_indices[b]].
 */
static void ssd_step_token(const problem *pb, int D_per_dim, double dt_min, double dt_max,
                           double *state, int64_t t, double *out) {
    const int64_t H = pb->nheads, P = pb->headdim, N = pb->dstate;
    const int64_t ratio = H / pb->ngroups;
    for (int64_t h = 0; h < H; ++h) {
        const int64_t grp = h / ratio;
        const double *Bt = pb->B + (t * pb->ngroups + grp) * N;
        const double *Ct = pb->C + (t * pb->ngroups + grp) * N;
        double u = pb->dt[t * H + h];
        if (pb->dt_bias) u += pb->dt_bias[h];
        if (pb->dt_softplus) u = softplus(u);
        u = fmin(fmax(u, dt_min), dt_max);
        const double decay = exp(pb->A[h] * u);
        for (int64_t p = 0; p < P; ++p) {
            const int64_t i = (t * H + h) * P + p;
            const double xv = pb->x[i];
            double *st = state + (h * P + p) * N;
            double dot = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                st[n] = st[n] * decay + u * Bt[n] * xv;
                dot += st[n] * Ct[n];
            }
            double y = dot;
            if (pb->D) y += (D_per_dim ? pb->D[h * P + p] : pb->D[h]) * xv;
            if (pb->z) y *= pb->z[i] * sigmoid(pb->z[i]);
            out[i] = y;
        }
    }
}

int oracle_ssd_prefill(int64_t tokens, int64_t nheads, int64_t headdim, int64_t dstate,
                       int64_t ngroups, const double *x, const double *dt, const double *A,
                       const double *B, const double *C, const double *D, int D_per_dim,
                       const double *z, const double *dt_bias, int dt_softplus,
                       double dt_min, double dt_max, int64_t chunk_size, int64_t nchunks,
                       const int64_t *cu_chunk_seqlens, const int64_t *seq_idx, int64_t batch,
                       const int64_t *last_chunk_indices, const double *initial_states,
                       double *out, double *chunk_states, double *final_states) {
    const problem pb = {1,      nheads, headdim, dstate,  ngroups, x, dt, A,
                        B,      C,      D,       z,       dt_bias, 0, dt_softplus};
    if (tokens < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0 || chunk_size <= 0 || nchunks < 1 || batch < 0)
        return -1;
    if (!cu_chunk_seqlens || !seq_idx || !chunk_states || (batch > 0 && !last_chunk_indices))
        return -1;
    if (tokens > 0 && (!x || !dt || !A || !B || !C || !out)) return -1;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t lo = cu_chunk_seqlens[c], hi = cu_chunk_seqlens[c + 1];
        if (lo < 0 || hi < lo || hi > tokens || hi - lo > chunk_size) return -1;
        if (initial_states && (seq_idx[c] < 0 || seq_idx[c] >= batch)) return -1;
    }
    for (int64_t b = 0; b < batch; ++b)
        if (last_chunk_indices[b] < 0 || last_chunk_indices[b] >= nchunks) return -1;

    const int64_t elems = nheads * headdim * dstate;
    double *s = (double *)calloc((size_t)elems, sizeof(double));
    if (!s) return -1;
    for (int64_t c = 0; c < nchunks; ++c) {
        if (c == 0 || seq_idx[c] != seq_idx[c - 1]) {
            if (initial_states)
                memcpy(s, initial_states + seq_idx[c] * elems, (size_t)elems * sizeof(double));
            else
                memset(s, 0, (size_t)elems * sizeof(double));
        }
        for (int64_t t = cu_chunk_seqlens[c]; t < cu_chunk_seqlens[c + 1]; ++t)
            ssd_step_token(&pb, D_per_dim, dt_min, dt_max, s, t, out);
        memcpy(chunk_states + c * elems, s, (size_t)elems * sizeof(double));
    }
    if (final_states)
        for (int64_t b = 0; b < batch; ++b)
            memcpy(final_states + b * elems, chunk_states + last_chunk_indices[b] * elems,
                   (size_t)elems * sizeof(double));
    free(s);
    return 0;
}
