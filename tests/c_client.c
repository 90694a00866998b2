/*
 * c_client.c -- drives the SSU C ABI from plain C, as a serving engine written
 * in C or C++ would: device buffers from hipMalloc, a HIP stream of its own, no
 * Python and no torch. One one-token call and one packed call, each checked
 * against the fp64 oracle (test infrastructure, linked here only):
 *   - out and the written states within max |gpu - ref| <= 1e-5 max(1, max |ref|)
 *     (fp32 state and io);
 *   - placement exact: slots the oracle leaves alone keep their bytes, and rows
 *     of inert sequences keep a NaN sentinel bit for bit.
 * A third call writes a bf16 state with stochastic rounding. Its expected bits
 * follow the layout include/ssu.h states for bf16 (Philox counter (e / 8, row,
 * 0), word (e % 8) / 2, its low half for even e and high half for odd e), built
 * here from the oracle's Philox and rounding rule on the oracle's unrounded
 * state; every stored value must equal that result except where the GPU's fp32
 * state sits next to a rounding threshold (at most 0.5 % of the elements, each
 * one bf16 step away).
 * A fourth call runs the SSD prefill (include/ssd.h) with a workspace of its
 * own, checked against the oracle's prefill at the same bars as the Python
 * tests (bf16 out within 1e-2 + 2e-2 |ref|, fp32 states within 1e-5 of their
 * scale).
 * Prints "c client ok" and exits 0 on success, 1 on a mismatch, 2 on a HIP or
 * library error.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssd.h"
#include "ssu.h"
#include "ssu_oracle.h"

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

enum { NSLOTS = 12, H = 4, P = 64, N = 128, G = 2 };
#define SLOT (H * P * N)
static const uint32_t kSentinel = 0x7FC0DEADu; /* a NaN no computation produces */

/* Seeded 64-bit LCG (Knuth's MMIX constants), top 53 bits as a uniform. */
static uint64_t rng_state = 0x243F6A8885A308D3ull;
static float uniform(float lo, float hi) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)(lo + (hi - lo) * ((double)(rng_state >> 11) * 0x1.0p-53));
}
static void fill(float* v, size_t n, float lo, float hi) {
    for (size_t i = 0; i < n; ++i) v[i] = uniform(lo, hi);
}
static double* widen(const float* v, size_t n) {
    double* d = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) d[i] = v[i];
    return d;
}
static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes));
    CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* bf16 <-> float by bit patterns: round to nearest even (finite inputs). */
static uint16_t bf16_bits(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* Per-head parameters shared by the calls. */
static float A[H], D[H], dt_bias[H];

/* Compare a GPU result with the oracle's. Returns the number of failures. */
static int compare(const char* what, int rows, const float* state0, const float* state_gpu,
                   const double* state_ref, const float* out_gpu, const double* out_ref,
                   const int* row_live) {
    int bad = 0;
    double scale = 1.0, err = 0.0;
    for (int s = 0; s < NSLOTS; ++s) {
        const size_t o = (size_t)s * SLOT;
        int touched = 0;
        for (size_t i = 0; i < SLOT && !touched; ++i) touched = state_ref[o + i] != (double)state0[o + i];
        if (!touched) {
            if (memcmp(state_gpu + o, state0 + o, SLOT * sizeof(float)) != 0) {
                fprintf(stderr, "%s: slot %d changed but the oracle leaves it alone\n", what, s);
                ++bad;
            }
            continue;
        }
        for (size_t i = 0; i < SLOT; ++i) {
            scale = fmax(scale, fabs(state_ref[o + i]));
            err = fmax(err, fabs((double)state_gpu[o + i] - state_ref[o + i]));
        }
    }
    if (err > 1e-5 * scale) {
        fprintf(stderr, "%s: state error %.3e at scale %.3e\n", what, err, scale);
        ++bad;
    }
    scale = 1.0;
    err = 0.0;
    for (int r = 0; r < rows; ++r) {
        const size_t o = (size_t)r * H * P;
        if (!row_live[r]) {
            for (size_t i = 0; i < H * P; ++i) {
                uint32_t bits;
                memcpy(&bits, out_gpu + o + i, sizeof bits);
                if (bits != kSentinel) {
                    fprintf(stderr, "%s: row %d of an inert sequence was written\n", what, r);
                    ++bad;
                    break;
                }
            }
            continue;
        }
        for (size_t i = 0; i < H * P; ++i) {
            scale = fmax(scale, fabs(out_ref[o + i]));
            err = fmax(err, fabs((double)out_gpu[o + i] - out_ref[o + i]));
        }
    }
    if (err > 1e-5 * scale) {
        fprintf(stderr, "%s: out error %.3e at scale %.3e\n", what, err, scale);
        ++bad;
    }
    printf("%s: %s\n", what, bad ? "MISMATCH" : "matches the oracle");
    return bad;
}

/* One call's operands on host and device; rows tokens. */
typedef struct {
    int rows;
    float *x, *z, *dt, *B, *C, *out;
    void *dx, *dz, *ddt, *dB, *dC, *dout;
} Tokens;

static Tokens make_tokens(int rows) {
    Tokens t;
    t.rows = rows;
    const size_t hp = (size_t)rows * H * P, gn = (size_t)rows * G * N;
    t.x = malloc(hp * sizeof(float));
    t.z = malloc(hp * sizeof(float));
    t.dt = malloc((size_t)rows * H * sizeof(float));
    t.B = malloc(gn * sizeof(float));
    t.C = malloc(gn * sizeof(float));
    t.out = malloc(hp * sizeof(float));
    fill(t.x, hp, -1.f, 1.f);
    fill(t.z, hp, -2.f, 2.f);
    fill(t.dt, (size_t)rows * H, -3.f, 0.f);
    fill(t.B, gn, -1.f, 1.f);
    fill(t.C, gn, -1.f, 1.f);
    for (size_t i = 0; i < hp; ++i) memcpy(&t.out[i], &kSentinel, sizeof(float));
    t.dx = to_device(t.x, hp * sizeof(float));
    t.dz = to_device(t.z, hp * sizeof(float));
    t.ddt = to_device(t.dt, (size_t)rows * H * sizeof(float));
    t.dB = to_device(t.B, gn * sizeof(float));
    t.dC = to_device(t.C, gn * sizeof(float));
    t.dout = to_device(t.out, hp * sizeof(float));
    return t;
}

static ssu_operands operands(void* dstate, const Tokens* t, const void* dA, const void* dD,
                             const void* dbias) {
    ssu_operands op;
    memset(&op, 0, sizeof op);
    op.state = dstate;
    op.state_dtype = SSU_F32;
    op.nslots = NSLOTS;
    op.nheads = H;
    op.headdim = P;
    op.dstate = N;
    op.ngroups = G;
    op.x = t->dx;
    op.B = t->dB;
    op.C = t->dC;
    op.z = t->dz;
    op.out = t->dout;
    op.io_dtype = SSU_F32;
    op.dt = t->ddt;
    op.A = dA;
    op.D = dD;
    op.dt_bias = dbias;
    op.dt_softplus = 1;
    op.pad_slot_id = -1;
    return op;
}

int main(void) {
    if (ssu_version() != SSU_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header %d\n", ssu_version(), SSU_ABI_VERSION);
        return 2;
    }
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    for (int h = 0; h < H; ++h) {
        A[h] = -expf(uniform(0.f, 2.f));
        D[h] = uniform(-1.f, 1.f);
        dt_bias[h] = uniform(-1.f, 1.f);
    }
    void* dA = to_device(A, sizeof A);
    void* dD = to_device(D, sizeof D);
    void* dbias = to_device(dt_bias, sizeof dt_bias);
    double *A64 = widen(A, H), *D64 = widen(D, H), *bias64 = widen(dt_bias, H);

    float* state0 = malloc((size_t)NSLOTS * SLOT * sizeof(float));
    fill(state0, (size_t)NSLOTS * SLOT, -1.f, 1.f);
    float* state_gpu = malloc((size_t)NSLOTS * SLOT * sizeof(float));
    double* state_ref = malloc((size_t)NSLOTS * SLOT * sizeof(double));
    double* state0_64 = widen(state0, (size_t)NSLOTS * SLOT);
    int failures = 0;

    /* ---- one token per sequence: sequence 2 reads a pad slot (inert); every
       sequence writes a slot no sequence reads. */
    {
        enum { BATCH = 5 };
        const int32_t src[BATCH] = {3, 7, -1, 0, 9};
        const int32_t dst[BATCH] = {4, 8, 5, 1, 10};
        const int live[BATCH] = {1, 1, 0, 1, 1};
        Tokens t = make_tokens(BATCH);
        void* dstate = to_device(state0, (size_t)NSLOTS * SLOT * sizeof(float));
        void* dsrc = to_device(src, sizeof src);
        void* ddst = to_device(dst, sizeof dst);
        ssu_one_token_args a;
        memset(&a, 0, sizeof a);
        a.struct_size = sizeof a;
        a.op = operands(dstate, &t, dA, dD, dbias);
        a.batch = BATCH;
        a.src_slots = dsrc;
        a.src_dtype = SSU_I32;
        a.dst_slots = ddst;
        a.dst_dtype = SSU_I32;
        if (ssu_one_token(&a, stream) != SSU_OK) {
            fprintf(stderr, "ssu_one_token: %s\n", ssu_last_error());
            return 2;
        }
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(state_gpu, dstate, (size_t)NSLOTS * SLOT * sizeof(float), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(t.out, t.dout, (size_t)BATCH * H * P * sizeof(float), hipMemcpyDeviceToHost));

        int64_t src64[BATCH], dst64[BATCH];
        for (int b = 0; b < BATCH; ++b) src64[b] = src[b], dst64[b] = dst[b];
        double* out_ref = malloc((size_t)BATCH * H * P * sizeof(double));
        double *x64 = widen(t.x, (size_t)BATCH * H * P), *z64 = widen(t.z, (size_t)BATCH * H * P);
        double *dt64 = widen(t.dt, (size_t)BATCH * H), *B64 = widen(t.B, (size_t)BATCH * G * N);
        double* C64 = widen(t.C, (size_t)BATCH * G * N);
        if (oracle_ssu_one_token(state0_64, state_ref, NSLOTS, H, P, N, G, BATCH, x64, dt64, 0, A64,
                                 B64, C64, D64, z64, bias64, 1, src64, dst64, -1, 0, NULL, out_ref) != 0) {
            fprintf(stderr, "oracle_ssu_one_token refused its arguments\n");
            return 2;
        }
        failures += compare("one-token", BATCH, state0, state_gpu, state_ref, t.out, out_ref, live);
    }

    /* ---- packed: three sequences of 3, 0 and 4 tokens; the acceptance count
       picks the read entry of a shared [3, 4] table, every token writes its own
       entry (-1 entries drop the write). */
    {
        enum { NSEQ = 3, STEPS = 4, ROWS = 7 };
        const int32_t cu[NSEQ + 1] = {0, 3, 3, 7};
        const int32_t accepted[NSEQ] = {2, 1, 3};
        const int32_t table[NSEQ * STEPS] = {2, 6, 11, -1, 1, 3, 4, 5, 0, 8, 9, 10};
        const int live[ROWS] = {1, 1, 1, 1, 1, 1, 1};
        Tokens t = make_tokens(ROWS);
        void* dstate = to_device(state0, (size_t)NSLOTS * SLOT * sizeof(float));
        void* dcu = to_device(cu, sizeof cu);
        void* dacc = to_device(accepted, sizeof accepted);
        void* dtab = to_device(table, sizeof table);
        ssu_packed_args a;
        memset(&a, 0, sizeof a);
        a.struct_size = sizeof a;
        a.op = operands(dstate, &t, dA, dD, dbias);
        a.rows = ROWS;
        a.nseq = NSEQ;
        a.cu_seqlens = dcu;
        a.num_accepted = dacc;
        a.meta_dtype = SSU_I32;
        a.src_table = dtab;
        a.src_dtype = SSU_I32;
        a.src_seq_stride = STEPS;
        a.src_step_stride = 1;
        a.dst_table = dtab;
        a.dst_dtype = SSU_I32;
        a.dst_seq_stride = STEPS;
        a.dst_step_stride = 1;
        a.steps = STEPS;
        if (ssu_packed_varlen(&a, stream) != SSU_OK) {
            fprintf(stderr, "ssu_packed_varlen: %s\n", ssu_last_error());
            return 2;
        }
        CHECK_HIP(hipStreamSynchronize(stream));
        CHECK_HIP(hipMemcpy(state_gpu, dstate, (size_t)NSLOTS * SLOT * sizeof(float), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(t.out, t.dout, (size_t)ROWS * H * P * sizeof(float), hipMemcpyDeviceToHost));

        int64_t cu64[NSEQ + 1], acc64[NSEQ], tab64[NSEQ * STEPS];
        for (int i = 0; i <= NSEQ; ++i) cu64[i] = cu[i];
        for (int i = 0; i < NSEQ; ++i) acc64[i] = accepted[i];
        for (int i = 0; i < NSEQ * STEPS; ++i) tab64[i] = table[i];
        double* out_ref = malloc((size_t)ROWS * H * P * sizeof(double));
        double *x64 = widen(t.x, (size_t)ROWS * H * P), *z64 = widen(t.z, (size_t)ROWS * H * P);
        double *dt64 = widen(t.dt, (size_t)ROWS * H), *B64 = widen(t.B, (size_t)ROWS * G * N);
        double* C64 = widen(t.C, (size_t)ROWS * G * N);
        if (oracle_ssu_packed_varlen(state0_64, state_ref, NSLOTS, H, P, N, G, ROWS, NSEQ, cu64, acc64,
                                     tab64, STEPS, 1, tab64, STEPS, 1, STEPS, x64, dt64, 0, A64, B64,
                                     C64, D64, z64, bias64, 1, -1, 0, NULL, out_ref) != 0) {
            fprintf(stderr, "oracle_ssu_packed_varlen refused its arguments\n");
            return 2;
        }
        failures += compare("packed", ROWS, state0, state_gpu, state_ref, t.out, out_ref, live);
    }

    /* ---- bf16 state, stochastic rounding: four sequences, each writing a slot
       no sequence reads. */
    {
        enum { BATCH = 4 };
        const int32_t src[BATCH] = {2, 6, 11, 0};
        const int32_t dst[BATCH] = {3, 7, 10, 1};
        const int64_t seed = 0x1234ABCD5678EF01ll;
        const int rounds = 10;
        const size_t elems = (size_t)NSLOTS * SLOT;
        uint16_t* s16 = malloc(elems * sizeof(uint16_t));
        double* s16_64 = malloc(elems * sizeof(double));
        for (size_t i = 0; i < elems; ++i) {
            s16[i] = bf16_bits(state0[i]);
            s16_64[i] = bf16_value(s16[i]);
        }
        Tokens t = make_tokens(BATCH);
        void* dstate = to_device(s16, elems * sizeof(uint16_t));
        void* dsrc = to_device(src, sizeof src);
        void* ddst = to_device(dst, sizeof dst);
        void* dseed = to_device(&seed, sizeof seed);
        ssu_one_token_args a;
        memset(&a, 0, sizeof a);
        a.struct_size = sizeof a;
        a.op = operands(dstate, &t, dA, dD, dbias);
        a.op.state_dtype = SSU_BF16;
        a.op.rand_seed = dseed;
        a.op.philox_rounds = rounds;
        a.batch = BATCH;
        a.src_slots = dsrc;
        a.src_dtype = SSU_I32;
        a.dst_slots = ddst;
        a.dst_dtype = SSU_I32;
        if (ssu_one_token(&a, stream) != SSU_OK) {
            fprintf(stderr, "ssu_one_token (bf16, stochastic rounding): %s\n", ssu_last_error());
            return 2;
        }
        CHECK_HIP(hipStreamSynchronize(stream));
        uint16_t* g16 = malloc(elems * sizeof(uint16_t));
        CHECK_HIP(hipMemcpy(g16, dstate, elems * sizeof(uint16_t), hipMemcpyDeviceToHost));

        int64_t src64[BATCH], dst64[BATCH];
        for (int b = 0; b < BATCH; ++b) src64[b] = src[b], dst64[b] = dst[b];
        double* ref = malloc(elems * sizeof(double));
        double* out_ref = malloc((size_t)BATCH * H * P * sizeof(double));
        double *x64 = widen(t.x, (size_t)BATCH * H * P), *z64 = widen(t.z, (size_t)BATCH * H * P);
        double *dt64 = widen(t.dt, (size_t)BATCH * H), *B64 = widen(t.B, (size_t)BATCH * G * N);
        double* C64 = widen(t.C, (size_t)BATCH * G * N);
        /* The unrounded fp64 states: no rounding argument. */
        if (oracle_ssu_one_token(s16_64, ref, NSLOTS, H, P, N, G, BATCH, x64, dt64, 0, A64, B64,
                                 C64, D64, z64, bias64, 1, src64, dst64, -1, 0, NULL, out_ref) != 0) {
            fprintf(stderr, "oracle_ssu_one_token refused its arguments\n");
            return 2;
        }
        const uint32_t key[2] = {(uint32_t)seed, (uint32_t)((uint64_t)seed >> 32)};
        long flips = 0, bad = 0, written = 0;
        for (int b = 0; b < BATCH; ++b) {
            const size_t o = (size_t)dst[b] * SLOT;
            for (uint32_t e = 0; e < SLOT; ++e) {
                /* The header's bf16 layout: row b's counter (e / 8, b, 0, 0). */
                const uint32_t ctr[4] = {e / 8, (uint32_t)b, 0u, 0u};
                uint32_t words[4];
                oracle_philox4x32(ctr, key, rounds, words);
                const uint32_t word = words[(e % 8) / 2];
                const uint32_t bits = (e % 2) ? (word >> 16) : (word & 0xFFFFu);
                const uint32_t w = bits << 16; /* the rounding reads the word's top bits */
                double want;
                oracle_round_stochastic(&ref[o + e], &w, 1, 2, &want);
                const double got = bf16_value(g16[o + e]);
                ++written;
                if (got == want) continue;
                /* The other neighbour, decided by the fp32 state near a threshold. */
                const double step = fabs(want) * 0x1p-7;
                if (fabs(got - want) <= step * 1.0000001 && fabs(got - ref[o + e]) <= step) ++flips;
                else ++bad;
            }
        }
        /* Slots no call writes keep their bytes. */
        for (int s = 0; s < NSLOTS; ++s) {
            int written_slot = 0;
            for (int b = 0; b < BATCH; ++b) written_slot |= dst[b] == s;
            if (!written_slot && memcmp(g16 + (size_t)s * SLOT, s16 + (size_t)s * SLOT,
                                        SLOT * sizeof(uint16_t)) != 0) {
                fprintf(stderr, "bf16 SR: slot %d changed but no sequence writes it\n", s);
                ++bad;
            }
        }
        const int ok = bad == 0 && flips * 200 <= written;
        printf("bf16 stochastic rounding: %ld of %ld elements match the header's layout, "
               "%ld threshold flips, %ld mismatches: %s\n", written - flips - bad, written,
               flips, bad, ok ? "matches" : "MISMATCH");
        failures += !ok;
    }

    /* ---- the SSD prefill (include/ssd.h): two requests of 150 and 40 tokens in
       chunks of 128 (three chunks), bf16 io, fp32 states, initial states, gate,
       D and dt_bias, and a workspace from hipMalloc of ssu_ssd_workspace_bytes.
       out and the per-request final states against the oracle at the bars:
       |err| <= 1e-2 + 2e-2 |ref| for bf16 out, max |err| <= 1e-5 max(1, max |ref|)
       for the fp32 states. */
    {
        enum { SH = 2, SP = 64, SN = 64, SG = 1, Q = 128, TOK = 190, NCH = 3, NB = 2 };
        const int32_t cu[NCH + 1] = {0, 128, 150, 190};
        const int32_t sidx[NCH] = {0, 0, 1};
        const int32_t last[NB] = {1, 2};
        const size_t nx = (size_t)TOK * SH * SP, nb = (size_t)TOK * SG * SN,
                     ns = (size_t)NB * SH * SP * SN;
        uint16_t *x16 = malloc(nx * 2), *z16 = malloc(nx * 2), *b16 = malloc(nb * 2),
                 *c16 = malloc(nb * 2), *o16 = malloc(nx * 2);
        double *x64 = malloc(nx * 8), *z64 = malloc(nx * 8), *b64 = malloc(nb * 8),
               *c64 = malloc(nb * 8);
        for (size_t i = 0; i < nx; ++i) {
            x16[i] = bf16_bits(uniform(-1.5f, 1.5f));
            x64[i] = bf16_value(x16[i]);
            z16[i] = bf16_bits(uniform(-2.f, 2.f));
            z64[i] = bf16_value(z16[i]);
        }
        for (size_t i = 0; i < nb; ++i) {
            b16[i] = bf16_bits(uniform(-1.5f, 1.5f));
            b64[i] = bf16_value(b16[i]);
            c16[i] = bf16_bits(uniform(-1.5f, 1.5f));
            c64[i] = bf16_value(c16[i]);
        }
        float dt[TOK * SH], a2[SH], d2[SH], bias2[SH];
        fill(dt, TOK * SH, -3.f, 0.f);
        for (int h = 0; h < SH; ++h) {
            a2[h] = -expf(uniform(0.f, 2.f));
            d2[h] = uniform(-1.f, 1.f);
            bias2[h] = uniform(-1.f, 1.f);
        }
        float* init = malloc(ns * sizeof(float));
        fill(init, ns, -1.f, 1.f);

        void *dx = to_device(x16, nx * 2), *dz = to_device(z16, nx * 2), *dB = to_device(b16, nb * 2),
             *dC = to_device(c16, nb * 2), *ddt = to_device(dt, sizeof dt),
             *dA2 = to_device(a2, sizeof a2), *dD2 = to_device(d2, sizeof d2),
             *dbias2 = to_device(bias2, sizeof bias2), *dinit = to_device(init, ns * sizeof(float)),
             *dcu = to_device(cu, sizeof cu), *dsidx = to_device(sidx, sizeof sidx),
             *dlast = to_device(last, sizeof last);
        void *dout = NULL, *dstates = NULL, *dwork = NULL;
        CHECK_HIP(hipMalloc(&dout, nx * 2));
        CHECK_HIP(hipMalloc(&dstates, ns * sizeof(float)));
        const size_t wbytes = ssu_ssd_workspace_bytes(NCH, NB, SH, SP, SN, SG, Q);
        CHECK_HIP(hipMalloc(&dwork, wbytes));

        ssu_ssd_args a;
        memset(&a, 0, sizeof a);
        a.struct_size = sizeof a;
        a.tokens = TOK;
        a.nheads = SH;
        a.headdim = SP;
        a.dstate = SN;
        a.ngroups = SG;
        a.chunk_size = Q;
        a.nchunks = NCH;
        a.batch = NB;
        a.x = dx;
        a.dt = ddt;
        a.A = dA2;
        a.B = dB;
        a.C = dC;
        a.D = dD2;
        a.z = dz;
        a.dt_bias = dbias2;
        a.io_dtype = SSU_BF16;
        a.dt_dtype = SSU_F32;
        a.dt_softplus = 1;
        a.dt_min = 0.0;
        a.dt_max = INFINITY;
        a.cu_chunk_seqlens = dcu;
        a.seq_idx = dsidx;
        a.last_chunk_indices = dlast;
        a.meta_dtype = SSU_I32;
        a.state_dtype = SSU_F32;
        a.initial_states = dinit;
        a.out = dout;
        a.states = dstates;
        a.workspace = dwork;
        a.workspace_bytes = wbytes;
        if (ssu_ssd_prefill(&a, stream) != SSU_OK) {
            fprintf(stderr, "ssu_ssd_prefill: %s\n", ssu_last_error());
            return 2;
        }
        CHECK_HIP(hipStreamSynchronize(stream));
        float* states_gpu = malloc(ns * sizeof(float));
        CHECK_HIP(hipMemcpy(o16, dout, nx * 2, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(states_gpu, dstates, ns * sizeof(float), hipMemcpyDeviceToHost));

        int64_t cu64[NCH + 1], sidx64[NCH], last64[NB];
        for (int c = 0; c <= NCH; ++c) cu64[c] = cu[c];
        for (int c = 0; c < NCH; ++c) sidx64[c] = sidx[c];
        for (int b = 0; b < NB; ++b) last64[b] = last[b];
        double *dt64 = widen(dt, TOK * SH), *a64 = widen(a2, SH), *d64 = widen(d2, SH),
               *bias64b = widen(bias2, SH), *init64 = widen(init, ns);
        double* out_ref = malloc(nx * 8);
        double* chunk_ref = malloc((size_t)NCH * SH * SP * SN * 8);
        double* final_ref = malloc(ns * 8);
        if (oracle_ssd_prefill(TOK, SH, SP, SN, SG, x64, dt64, a64, b64, c64, d64, 0, z64, bias64b,
                               1, 0.0, INFINITY, Q, NCH, cu64, sidx64, NB, last64, init64, out_ref,
                               chunk_ref, final_ref) != 0) {
            fprintf(stderr, "oracle_ssd_prefill refused its arguments\n");
            return 2;
        }
        long bad_out = 0;
        double worst_out = 0.0;
        for (size_t i = 0; i < nx; ++i) {
            const double err = fabs((double)bf16_value(o16[i]) - out_ref[i]);
            const double bar = 1e-2 + 2e-2 * fabs(out_ref[i]);
            if (!(err <= bar)) ++bad_out;
            if (err / bar > worst_out) worst_out = err / bar;
        }
        double scale = 1.0, worst_st = 0.0;
        for (size_t i = 0; i < ns; ++i) scale = fmax(scale, fabs(final_ref[i]));
        for (size_t i = 0; i < ns; ++i) worst_st = fmax(worst_st, fabs(states_gpu[i] - final_ref[i]));
        const int ok = bad_out == 0 && worst_st <= 1e-5 * scale;
        printf("ssd prefill: out worst err/bar %.3f (%ld outside), final states max err %.2e "
               "(bar %.2e): %s\n", worst_out, bad_out, worst_st, 1e-5 * scale,
               ok ? "matches the oracle" : "MISMATCH");
        failures += !ok;
        void* bufs[] = {dx, dz, dB, dC, ddt, dA2, dD2, dbias2, dinit, dcu, dsidx, dlast,
                        dout, dstates, dwork};
        for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
        free(x16); free(z16); free(b16); free(c16); free(o16); free(x64); free(z64); free(b64);
        free(c64); free(init); free(states_gpu); free(dt64); free(a64); free(d64); free(bias64b);
        free(init64); free(out_ref); free(chunk_ref); free(final_ref);
    }

    CHECK_HIP(hipStreamDestroy(stream));
    if (failures) return 1;
    printf("c client ok\n");
    return 0;
}
