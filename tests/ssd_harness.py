"""SSD prefill: the GPU call, the oracle on the same inputs, and the comparison.

Tolerances (the bar the decode step is held to, applied unchanged):
  16-bit results (out, and fp16/bf16 states): |gpu - ref| <= 1e-2 + 2e-2 |ref|
      element by element;
  fp32 states: max |gpu - ref| <= 1e-5 max(1, max |ref|) over the compared tensor.

Beside the bar each check reports a diagnostic: the error against the size of
the terms that make up each result, err / (2^-14 mag + u |ref|), where mag is
the same recurrence run on |x|, |B|, |C|, |D|, |initial state| (every decay and
step is positive) times |z sigmoid(z)|, and u the result type's spacing at 1
(the final rounding). The matrix-core products take 16-bit operands and
accumulate in fp32; x, B and C enter exactly and every derived operand (decayed
C B^T entry, weighted x, entering state) as a high and a low 16-bit part, so a
bf16 product is off by about 2^-16 of its terms and the diagnostic stays near or
below one for bf16 io (an operand that lost its low part shows as a value of
tens). With fp16 io the low parts of small values fall into fp16's subnormals,
an absolute error of up to 2^-25 per term that the relative diagnostic does not
model, so its values there are larger while the bar still holds.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -24}


def np64(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def npi(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.int64)


def run_gpu(w, out=None):
    import selective_state_update_ssu_amd as ssu
    states = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())
    return out, states


def oracle_ref(w, orc=None):
    """(ref, mag): oracle results on the workload's exact inputs, and the
    magnitude run (absolute values) for the tolerance."""
    orc = orc or oracle.default()
    x, dt, A, B, C = (np64(t) for t in (w.x, w.dt, w.A, w.B, w.C))
    D, z, bias, init = (np64(t) for t in (w.D, w.z, w.dt_bias, w.initial_states))
    meta = [npi(t) for t in (w.cu_chunk_seqlens, w.seq_idx, w.last_chunk_indices)]
    common = dict(dt_bias=bias, dt_softplus=w.dt_softplus, dt_limit=w.dt_limit)
    ref = orc.ssd_prefill(x, dt, A, B, C, w.chunk_size, *meta, D=D, z=z, initial_states=init,
                          **common)
    mag = orc.ssd_prefill(np.abs(x), dt, A, np.abs(B), np.abs(C), w.chunk_size, *meta,
                          D=None if D is None else np.abs(D), z=None,
                          initial_states=None if init is None else np.abs(init), **common)
    if z is not None:
        mag.out *= np.abs(z / (1.0 + np.exp(-z)))
    return ref, mag


def _report(err, tol, what):
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = float(np.max(err / tol))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance "
                             f"(worst err/tol {ratio:.2f}); first at {idx.tolist()}")


def bar_tolerance(ref, dtype):
    """The tolerance array of the bar for results stored in `dtype`."""
    if dtype == torch.float32:
        return np.full(ref.shape, 1e-5 * max(1.0, float(np.max(np.abs(ref), initial=0.0))))
    return 1e-2 + 2e-2 * np.abs(ref)


def diagnostic(err, ref, mag, dtype):
    """err / (2^-14 mag + u |ref| + 1e-30): the error against the terms' size."""
    return float(np.max(err / (2.0 ** -14 * mag + UNIT[dtype] * np.abs(ref) + 1e-30),
                        initial=0.0))


def check_out(gpu_out, ref_out, mag_out, io_dtype, rows=None, what="out"):
    """Every element of out within the bar; returns (worst err / bar, diagnostic)."""
    g = np64(gpu_out)
    if rows is not None:
        g, ref_out, mag_out = g[rows], ref_out[rows], mag_out[rows]
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - ref_out)
    tol = bar_tolerance(ref_out, io_dtype)
    _report(err, tol, what)
    return float(np.max(err / tol, initial=0.0)), diagnostic(err, ref_out, mag_out, io_dtype)


def check_states(gpu_states, ref_states, mag_states, state_dtype, io_dtype=None, what="states"):
    """Returned states within the bar of their type; returns (worst err / bar,
    diagnostic)."""
    g = np64(gpu_states)
    assert g.shape == ref_states.shape, (what, g.shape, ref_states.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - ref_states)
    tol = bar_tolerance(ref_states, state_dtype)
    _report(err, tol, what)
    return (float(np.max(err / tol, initial=0.0)),
            diagnostic(err, ref_states, mag_states, state_dtype))


def check_all(w, gpu_out, gpu_states, ref, mag):
    """Every row of out and every returned state; returns the (worst err / bar,
    diagnostic) pairs of both."""
    r_out = check_out(gpu_out, ref.out, mag.out, w.x.dtype)
    if w.return_intermediate_states:
        r_st = check_states(gpu_states, ref.chunk_states, mag.chunk_states, w.state_dtype,
                            w.x.dtype, "chunk states")
    else:
        r_st = check_states(gpu_states, ref.final_states, mag.final_states, w.state_dtype,
                            w.x.dtype, "final states")
    return r_out, r_st


def cut_request(w, b, heads=None):
    """Request b alone (consistent chunk metadata assumed): its tokens, chunks
    and initial state, as a workload of one request on the CPU; with `heads`,
    only those heads, each with its group's B and C as a group of its own."""
    from selective_state_update_ssu_amd.workloads import SsdWorkload
    cu = npi(w.cu_seqlens)
    si = npi(w.seq_idx)
    cc = npi(w.cu_chunk_seqlens)
    lo, hi = int(cu[b]), int(cu[b + 1])
    chunks = np.nonzero(si == b)[0]
    c0, c1 = int(chunks[0]), int(chunks[-1])
    H, G = w.x.shape[1], w.B.shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    gs = [h // (H // G) for h in hs] if heads is not None else list(range(G))
    hsel = lambda t, dim: None if t is None else t.cpu().index_select(dim, torch.tensor(hs))
    sl = lambda t: None if t is None else t[lo:hi].cpu()
    meta = lambda v: torch.tensor(v, dtype=torch.int64)
    init = None
    if w.initial_states is not None:
        init = hsel(w.initial_states[b:b + 1], 1)
    cut = SsdWorkload(
        name=f"{w.name}[{b}]", x=hsel(sl(w.x), 1), dt=hsel(sl(w.dt), 1), A=hsel(w.A, 0),
        B=sl(w.B)[:, gs], C=sl(w.C)[:, gs], chunk_size=w.chunk_size,
        cu_seqlens=meta([0, hi - lo]), cu_chunk_seqlens=meta(cc[c0:c1 + 2] - lo),
        seq_idx=meta([0] * (c1 - c0 + 1)), last_chunk_indices=meta([c1 - c0]),
        state_dtype=w.state_dtype, D=hsel(w.D, 0), z=hsel(sl(w.z), 1),
        dt_bias=hsel(w.dt_bias, 0), initial_states=init, dt_softplus=w.dt_softplus,
        dt_limit=w.dt_limit)
    return cut, (lo, hi), hs
