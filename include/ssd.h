/*
 * ssd.h -- C ABI of the SSD chunked prefill on MI355X (gfx950), the step that
 * runs a Mamba-2 layer over whole prompts and leaves the state the decode-time
 * update (ssu.h) continues from. Part of the same library as ssu.h; errors are
 * reported through ssu_last_error().
 *
 * Contract: the MATE documentation page "Source code for mate.mamba",
 * `ssd_combined_fwd_varlen` (its docstring and argument checks), which matches
 * vLLM's Mamba-2 prefill caller:
 *   - tokens of all requests are packed: x, z, out [tokens, nheads, headdim];
 *     dt [tokens, nheads]; B, C [tokens, ngroups, dstate];
 *   - chunk c covers tokens [cu_chunk_seqlens[c], cu_chunk_seqlens[c+1]); a chunk
 *     never spans two requests and holds at most chunk_size tokens (every chunk
 *     but a request's last holds exactly chunk_size);
 *   - seq_idx[c] is the request owning chunk c. A chunk opens a request when it
 *     is the first chunk or its seq_idx differs from the previous chunk's; that
 *     transition, not last_chunk_indices, decides where the entering state
 *     comes from: an opening chunk enters with initial_states[seq_idx[c]] (zeros
 *     without initial states), any other chunk with the state the previous chunk
 *     left;
 *   - the returned states are every chunk's final state [nchunks, nheads,
 *     headdim, dstate] when return_intermediate_states is set, otherwise
 *     states[last_chunk_indices[b]] for each request b, [batch, nheads, headdim,
 *     dstate]; both in state_dtype.
 * The arithmetic is the Mamba-2 recurrence the chunked algorithm equals (Dao &
 * Gu, "Transformers are SSMs", ICML 2024, sections 5 and 6), token by token
 * inside each request:
 *     v  = dt[t, h] (+ dt_bias[h]);  v = softplus(v) if dt_softplus;
 *     v  = min(max(v, dt_min), dt_max)
 *     s  = s * exp(A[h] v) + v * B[t, g] x[t, h, p]        (g = h / (nheads/ngroups))
 *     y  = C[t, g] . s + D x[t, h, p];  y *= z sigmoid(z) if z is given
 *     out[t, h, p] = y
 * The GPU computes it by chunks (intra-chunk products, and the state carried
 * from chunk to chunk along each request) on the matrix cores with 16-bit
 * operands and fp32 accumulation. x, B and C enter those products exactly; every
 * derived operand (the decayed C B^T entries, the weighted x, the state handed
 * from one chunk to the next) enters as a high and a low 16-bit part, so each
 * product is accurate to about 2^-16 of itself and the results agree with the
 * recurrence to within the final rounding of out and of the states (tolerances:
 * 16-bit |err| <= 1e-2 + 2e-2 |ref|, fp32 states max |err| <= 1e-5 max(1,
 * max |ref|)). With fp16 io the decayed C B^T entries and the states must stay
 * within fp16's range.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#include "ssu.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssu_ssd_args {
    uint32_t struct_size;       /* sizeof(ssu_ssd_args) */
    int64_t tokens;             /* rows of x, dt, B, C, z, out; >= 0 */
    int64_t nheads, headdim, dstate, ngroups;  /* nheads % ngroups == 0 */
    int64_t chunk_size;         /* most tokens a chunk may hold */
    int64_t nchunks;            /* >= 1 */
    int64_t batch;              /* requests: rows of initial_states and of the
                                   per-request returned states; >= 0 */
    /* Operands (device pointers, row-major, contiguous; x, B, C, z and out
       16-byte aligned). */
    const void *x;              /* [tokens, nheads, headdim] io_dtype */
    const void *dt;             /* [tokens, nheads] dt_dtype */
    const float *A;             /* [nheads] */
    const void *B;              /* [tokens, ngroups, dstate] io_dtype */
    const void *C;              /* [tokens, ngroups, dstate] io_dtype */
    const float *D;             /* [nheads] or [nheads, headdim] (D_per_dim), or NULL */
    const void *z;              /* [tokens, nheads, headdim] io_dtype, or NULL */
    const float *dt_bias;       /* [nheads] or NULL */
    int32_t io_dtype;           /* SSU_F16 or SSU_BF16: x, B, C, z, out */
    int32_t dt_dtype;           /* SSU_F32, SSU_F16 or SSU_BF16 */
    int32_t D_per_dim;          /* D is [nheads, headdim] */
    int32_t dt_softplus;
    double dt_min, dt_max;      /* dt_limit; (0, +inf) by default */
    /* Chunk metadata (device, meta_dtype). */
    const void *cu_chunk_seqlens;    /* [nchunks + 1] */
    const void *seq_idx;             /* [nchunks] */
    const void *last_chunk_indices;  /* [batch] */
    int32_t meta_dtype;              /* SSU_I32 or SSU_I64 */
    int32_t state_dtype;             /* SSU_F32, SSU_F16 or SSU_BF16 */
    const void *initial_states;      /* [batch, nheads, headdim, dstate] state_dtype, or NULL */
    void *out;                       /* [tokens, nheads, headdim] io_dtype, written */
    void *states;                    /* returned states (see above), state_dtype, written;
                                        16-byte aligned */
    int32_t return_intermediate_states;
    int32_t reserved;                /* 0 */
    /* Scratch owned by the caller, 256-byte aligned, at least
       ssu_ssd_workspace_bytes(...) bytes; its contents on entry do not matter. */
    void *workspace;
    size_t workspace_bytes;
} ssu_ssd_args;

/* Bytes of workspace ssu_ssd_prefill needs for these sizes: each chunk's
 * entering state as io-type high parts and 8-bit low parts (three bytes per
 * element), the per-chunk C B^T products
 * (fp32), each chunk's
 * steps, running sums, weights and decay per head, the chunk descriptors, the
 * per-request list of last chunks and the runs of chunks that continue one
 * another. Linear in nchunks; no term grows with the number of tokens beyond
 * nchunks * chunk_size. */
size_t ssu_ssd_workspace_bytes(int64_t nchunks, int64_t batch, int64_t nheads,
                               int64_t headdim, int64_t dstate, int64_t ngroups,
                               int64_t chunk_size);

/*
 * The whole prefill as kernel launches on `stream` (a hipStream_t; NULL is the
 * null stream): no allocation, no host-device copy, no synchronisation. Rows of
 * out that no chunk covers are not written.
 *
 * Returns SSU_OK, SSU_ERR_INVALID_ARGUMENT (inconsistent sizes or dtypes, a null
 * required pointer, out overlapping an input, a workspace too small or
 * misaligned), SSU_ERR_UNSUPPORTED (a headdim / dstate / chunk_size without
 * compiled kernels -- headdim 64, 128, 192 or 256, dstate 64, 128 or 256,
 * chunk_size 128 or 256 -- or
 * a misaligned operand) or SSU_ERR_LAUNCH.
 *
 * Device data is not validated by the host. Preconditions, as on the pages:
 * chunk ranges inside [0, tokens], in order and no longer than chunk_size;
 * seq_idx in [0, batch) where initial states are read; last_chunk_indices in
 * [0, nchunks). The kernels stay in bounds when these fail: a chunk with a bad
 * range is treated as empty, a seq_idx out of range enters with zeros, and a
 * request whose last-chunk index is out of range gets no returned state.
 */
int ssu_ssd_prefill(const ssu_ssd_args *args, void *stream);

/* Bytes of the static scratch ssu_ssd_prefill_noalloc uses on each GPU. */
#define SSU_SSD_STATIC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * ssu_ssd_prefill without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The caller still owns
 * every input and output; args->workspace must be NULL and workspace_bytes 0.
 * The scratch is a static array of SSU_SSD_STATIC_SCRATCH_BYTES (128 MiB) in the
 * library's device code: each GPU the library runs on holds one until the
 * process ends, and its address is looked up on the entry point's first call on
 * a device (make the stream's device current, as for every HIP call). Calls
 * that overlap in time on one GPU share that array and race: order them on one
 * stream (or use ssu_ssd_prefill with a workspace each). The array keeps the
 * last call's contents; no call needs it cleared.
 *
 * Returns what ssu_ssd_prefill returns, and SSU_ERR_UNSUPPORTED when the call's
 * workspace (ssu_ssd_workspace_bytes) exceeds SSU_SSD_STATIC_SCRATCH_BYTES
 * (it holds up to 34 chunks of 128 tokens at 128 heads x 64 x 128 with 8 groups,
 * 54 chunks of 256 at 80 heads x 64 x 128 with 1 group), SSU_ERR_LAUNCH when
 * no device is current or the scratch cannot be found on it. Results are those
 * of ssu_ssd_prefill, bit for bit (the same kernels).
 */
int ssu_ssd_prefill_noalloc(const ssu_ssd_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
