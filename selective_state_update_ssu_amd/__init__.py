"""Mamba-2 selective state update (SSU) decode step on AMD Instinct MI355X.

Python binding of the C ABI in include/ssu.h. It checks tensor shapes, dtypes,
devices and contiguity, then hands raw device pointers and torch's current HIP
stream to the library; every step of the update runs in the library's gfx950
kernel. There is no fallback: without the built library every call raises.

    ssu_one_token(state, x, dt, A, B, C, out=None, *, D, z, dt_bias, dt_softplus,
                  state_batch_indices, dst_state_batch_indices, pad_slot_id,
                  disable_state_update)
    ssu_packed_varlen(state, x, dt, A, B, C, cu_seqlens, out=None, *,
                      num_accepted_tokens, state_batch_indices,
                      dst_state_batch_indices, ...)
    prepare_one_token(...), prepare_packed_varlen(...)  -> PreparedCall
        (the same arguments, checked and marshalled once; call() relaunches)

    ssd_combined_fwd_varlen(x, dt, A, B, C, chunk_size, cu_seqlens,
                            cu_chunk_seqlens, last_chunk_indices, seq_idx, out=None, *,
                            D, z, dt_bias, dt_softplus, dt_limit, initial_states,
                            return_intermediate_states, state_dtype, workspace,
                            static_scratch)

Operand shapes follow the MATE documentation page "Source code for mate.mamba"
(`selective_state_update`): state [slots, heads, dim, dstate]; x, z, out
[rows, heads, dim]; dt [rows, heads], [rows, heads, 1] or [rows, heads, dim]
in fp32; B, C [rows, groups, dstate] in x's dtype; A, D, dt_bias fp32 [heads].
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import torch

from . import _abi

__all__ = ["ssu_one_token", "ssu_packed_varlen", "prepare_one_token", "prepare_packed_varlen",
           "PreparedCall", "update_replayssm_ring_trackers",
           "reset_replayssm_ring_trackers", "commit_replayssm_ring_trackers",
           "ssd_combined_fwd_varlen", "ssd_workspace_bytes", "reset_ssd_workspaces",
           "library_path", "library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBRARY = os.path.join(_HERE, "_lib", "libssu_amd.so")
_lib = None
_lock = threading.Lock()

_STATE_DTYPES = {torch.float32: _abi.SSU_F32, torch.float16: _abi.SSU_F16,
                 torch.bfloat16: _abi.SSU_BF16}
_IO_DTYPES = _STATE_DTYPES
_INDEX_DTYPES = {torch.int32: _abi.SSU_I32, torch.int64: _abi.SSU_I64}


def library_path() -> str:
    return _LIBRARY


def library() -> ctypes.CDLL:
    """The loaded HIP library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                _lib = _abi.load(_LIBRARY)
    return _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_device(device, **tensors):
    if device.type != "cuda":
        raise ValueError(f"state must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, state is on {device}")


def _contig(name, t):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _per_head(name, t, heads, dim=None, dstate=None):
    """One fp32 value per head. Besides a [heads] vector this accepts the tied
    views callers pass for a per-head parameter (MATE page, `_per_head`): a
    [heads, dim] or [heads, dim, dstate] tensor whose every dimension after the
    first has size 1 or stride 0 -- e.g. D[:, None].expand(heads, dim) or
    A[:, None, None].expand(heads, dim, dstate). Its first column is the
    per-head vector. A parameter that varies along dim or dstate is per channel,
    which this library does not implement."""
    if t is None:
        return None
    if t.dtype != torch.float32:
        raise NotImplementedError(f"{name} must be fp32, got {t.dtype}")
    if t.dim() not in (1, 2, 3) or t.shape[0] != heads:
        raise ValueError(f"{name} must be [{heads}], [{heads}, dim] or [{heads}, dim, dstate]; "
                         f"got {tuple(t.shape)}")
    for i, size in enumerate(t.shape[1:], start=1):
        want = dim if i == 1 else dstate
        if size != 1 and want is not None and size != want:
            raise ValueError(f"{name} dimension {i} has size {size}, expected 1 or {want}")
        if size != 1 and t.stride(i) != 0:
            raise NotImplementedError(
                f"{name} varies along dimension {i} (shape {tuple(t.shape)}, strides "
                f"{tuple(t.stride())}); only per-head values (size 1 or stride 0 there) are "
                f"implemented")
    while t.dim() > 1:
        t = t[..., 0]
    return t.contiguous()


def _seed(rand_seed, device):
    if rand_seed is None:
        return None
    if rand_seed.dtype != torch.int64 or rand_seed.numel() != 1:
        raise ValueError(f"rand_seed must be a one-element int64 tensor, got {rand_seed.dtype} "
                         f"{tuple(rand_seed.shape)}")
    if rand_seed.device != device:
        raise ValueError(f"rand_seed is on {rand_seed.device}, state is on {device}")
    return rand_seed


def _operands(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus, pad_slot_id,
              disable_state_update, heads_per_block, loads_per_lane, tile_order,
              rand_seed=None, philox_rounds=10):
    if state.dim() != 4:
        raise ValueError(f"state must be [slots, heads, dim, dstate], got {tuple(state.shape)}")
    if state.dtype not in _STATE_DTYPES:
        raise NotImplementedError(f"state dtype {state.dtype} is not supported")
    slots, heads, dim, dstate = state.shape
    if x.dim() != 3 or x.shape[1:] != (heads, dim):
        raise ValueError(f"x must be [rows, {heads}, {dim}], got {tuple(x.shape)}")
    rows = x.shape[0]
    if x.dtype not in _IO_DTYPES:
        raise NotImplementedError(f"x dtype {x.dtype} is not supported")
    if dt.dtype != torch.float32:
        raise NotImplementedError(f"dt must be fp32, got {dt.dtype}")
    if dt.shape == (rows, heads, dim) and dim > 1 and dt.stride(2) == 0:
        dt = dt[:, :, 0]  # one value per (row, head) broadcast along dim
    if dt.shape == (rows, heads) or dt.shape == (rows, heads, 1):
        dt_per_dim = 0
    elif dt.shape == (rows, heads, dim):
        dt_per_dim = 1
    else:
        raise ValueError(f"dt must be [rows, heads], [rows, heads, 1] or [rows, heads, dim]; "
                         f"got {tuple(dt.shape)}")
    if B.dim() != 3 or B.shape[0] != rows or B.shape[2] != dstate or C.shape != B.shape:
        raise ValueError(f"B/C must be [rows, groups, {dstate}]; got B={tuple(B.shape)}, "
                         f"C={tuple(C.shape)}")
    if B.dtype != x.dtype or C.dtype != x.dtype:
        raise ValueError("B and C must share the x dtype")
    groups = B.shape[1]
    if groups < 1 or heads % groups:
        raise ValueError(f"heads ({heads}) must be a multiple of groups ({groups})")
    if z is not None and (z.shape != x.shape or z.dtype != x.dtype):
        raise ValueError("z must match x in shape and dtype")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError(f"out must be {x.dtype} {tuple(x.shape)}, got {out.dtype} {tuple(out.shape)}")
    A = _per_head("A", A, heads, dim, dstate)
    D = _per_head("D", D, heads, dim, dstate)
    dt_bias = _per_head("dt_bias", dt_bias, heads, dim, dstate)
    _check_device(state.device, x=x, dt=dt, A=A, B=B, C=C, out=out, D=D, z=z, dt_bias=dt_bias)
    for name, t in (("state", state), ("x", x), ("dt", dt), ("B", B), ("C", C), ("z", z),
                    ("out", out)):
        _contig(name, t)
    op = _abi.Operands(
        state=_ptr(state), state_dtype=_STATE_DTYPES[state.dtype], nslots=slots, nheads=heads,
        headdim=dim, dstate=dstate, ngroups=groups,
        x=_ptr(x), B=_ptr(B), C=_ptr(C), z=_ptr(z), out=_ptr(out), io_dtype=_IO_DTYPES[x.dtype],
        dt=_ptr(dt), dt_per_dim=dt_per_dim, A=_ptr(A), D=_ptr(D), dt_bias=_ptr(dt_bias),
        dt_softplus=int(bool(dt_softplus)), pad_slot_id=int(pad_slot_id),
        disable_state_update=int(bool(disable_state_update)),
        rand_seed=_ptr(_seed(rand_seed, state.device)), philox_rounds=int(philox_rounds),
        heads_per_block=int(heads_per_block), loads_per_lane=int(loads_per_lane),
        tile_order=int(tile_order))
    # The temporaries whose pointers op holds stay referenced until the launch.
    return op, out, rows, (A, D, dt_bias, dt)


def _index(name, t, device):
    if t is None:
        return None, 0
    if t.dtype not in _INDEX_DTYPES:
        raise ValueError(f"{name} must be int32 or int64, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, state is on {device}")
    _contig(name, t)
    return t, _INDEX_DTYPES[t.dtype]


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a public call with `stream` (a torch.cuda.Stream, when given) as the
    current stream: the temporaries the binding makes (contiguous copies of
    per-head parameters, a missing out, workspace) are then allocated and
    written on the stream the kernels run on, so the caching allocator cannot
    hand their memory to other work while the kernels still read it. Inputs the
    caller produced on another stream must be ordered by the caller, as for any
    torch op."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def _raise(lib, rc, entry):
    msg = lib.ssu_last_error().decode(errors="replace")
    if rc == _abi.SSU_ERR_INVALID_ARGUMENT:
        raise ValueError(f"{entry}: {msg}")
    if rc == _abi.SSU_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{entry}: {msg}")
    raise RuntimeError(f"{entry}: {msg} (status {rc})")


@_on_stream
def ssu_one_token(state, x, dt, A, B, C, out=None, *, D=None, z=None, dt_bias=None,
                  dt_softplus=False, state_batch_indices=None, dst_state_batch_indices=None,
                  pad_slot_id=-1, disable_state_update=False, rand_seed=None,
                  philox_rounds=10, heads_per_block=0, loads_per_lane=0, tile_order=0,
                  stream=None):
    """One decode token per sequence (row b is sequence b). Updates `state` in place
    at the destination slots and returns `out` [batch, heads, dim].
    rand_seed (a one-element int64 device tensor) turns on stochastic rounding of
    stored fp16/bf16 states with Philox4x32-`philox_rounds`.
    heads_per_block / loads_per_lane / tile_order pick the launch shape (0: the
    library default)."""
    return _one_token_call(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus,
                           state_batch_indices, dst_state_batch_indices, pad_slot_id,
                           disable_state_update, rand_seed, philox_rounds, heads_per_block,
                           loads_per_lane, tile_order)(stream)


def _one_token_call(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus,
                    state_batch_indices, dst_state_batch_indices, pad_slot_id,
                    disable_state_update, rand_seed, philox_rounds, heads_per_block,
                    loads_per_lane, tile_order):
    op, out, batch, keep = _operands(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus,
                                     pad_slot_id, disable_state_update, heads_per_block,
                                     loads_per_lane, tile_order, rand_seed, philox_rounds)
    src, src_dt = _index("state_batch_indices", state_batch_indices, state.device)
    dst, dst_dt = _index("dst_state_batch_indices", dst_state_batch_indices, state.device)
    for name, t in (("state_batch_indices", src), ("dst_state_batch_indices", dst)):
        if t is not None and (t.dim() != 1 or t.shape[0] != batch):
            raise ValueError(f"{name} must be [{batch}], got {tuple(t.shape)}")
    args = _abi.OneTokenArgs(struct_size=ctypes.sizeof(_abi.OneTokenArgs), op=op, batch=batch,
                             src_slots=_ptr(src), src_dtype=src_dt,
                             dst_slots=_ptr(dst), dst_dtype=dst_dt)
    return PreparedCall("ssu_one_token", args, state.device, out,
                        (state, x, dt, B, C, z, src, dst, rand_seed) + keep)


class PreparedCall:
    """A decode call whose arguments were checked and marshalled once: calling it
    launches the update again on the same tensors (their current contents) and
    returns `out`. It keeps every tensor it points at alive. For decode loops
    that reuse their buffers from step to step, as graph-captured loops do: the
    per-call host work is one C call (see `prepare_one_token`)."""

    __slots__ = ("_entry", "_fn", "_args", "_ref", "_device", "out", "_keep")

    def __init__(self, entry, args, device, out, keep):
        self._entry, self._args, self._device, self.out, self._keep = entry, args, device, out, keep
        self._fn = getattr(library(), entry)
        self._ref = ctypes.byref(args)

    def __call__(self, stream=None):
        """Launch on `stream` (a torch.cuda.Stream; default: the current stream)."""
        s = torch.cuda.current_stream(self._device) if stream is None else stream
        rc = self._fn(self._ref, ctypes.c_void_p(s.cuda_stream))
        if rc != _abi.SSU_OK:
            _raise(library(), rc, self._entry)
        return self.out


def prepare_one_token(state, x, dt, A, B, C, out=None, *, D=None, z=None, dt_bias=None,
                      dt_softplus=False, state_batch_indices=None,
                      dst_state_batch_indices=None, pad_slot_id=-1,
                      disable_state_update=False, rand_seed=None, philox_rounds=10,
                      heads_per_block=0, loads_per_lane=0, tile_order=0):
    """`ssu_one_token`'s checks and marshalling, done once. Returns a
    PreparedCall; `call(stream=None)` runs the update on the tensors given here
    (their contents at the time of the call) and returns out. Temporaries are
    made now, on the current stream: a missing out, and contiguous copies of
    per-head parameters given as tied views (A, D and dt_bias are then read as
    they were at preparation, as model constants are)."""
    return _one_token_call(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus,
                           state_batch_indices, dst_state_batch_indices, pad_slot_id,
                           disable_state_update, rand_seed, philox_rounds, heads_per_block,
                           loads_per_lane, tile_order)


def _table(name, t, device, nseq):
    """(tensor, dtype code, seq stride, step stride, width) of a slot table."""
    t, code = _index(name, t, device)
    if t is None:
        return None, 0, 0, 0, None
    if t.dim() == 2:
        if t.shape[0] != nseq:
            raise ValueError(f"{name} must have one row per sequence ({nseq}), got {t.shape[0]}")
        return t, code, t.stride(0), t.stride(1), t.shape[1]
    if t.dim() == 1:
        # Flat per-row form: sequence b's position t is entry b + t.
        return t, code, 1, 1, t.shape[0] - nseq + 1
    raise ValueError(f"{name} must be [sequences, steps] or flat [rows], got {tuple(t.shape)}")


def _flatten_dense(name, t, lead, min_dim=4):
    """[batch, steps, ...] -> [batch * steps, ...] (a view for contiguous input)."""
    if t is None:
        return None
    if t.dim() < min_dim or tuple(t.shape[:2]) != lead:
        raise ValueError(f"a dense x [{lead[0]}, {lead[1]}, heads, dim] needs {name} in the "
                         f"same layout, got {tuple(t.shape)}")
    return t.reshape(lead[0] * lead[1], *t.shape[2:])


@_on_stream
def ssu_packed_varlen(state, x, dt, A, B, C, cu_seqlens=None, out=None, *,
                      num_accepted_tokens=None, state_batch_indices=None,
                      dst_state_batch_indices=None, D=None, z=None, dt_bias=None,
                      dt_softplus=False, pad_slot_id=-1, disable_state_update=False,
                      rand_seed=None, philox_rounds=10, steps=None, heads_per_block=0,
                      loads_per_lane=0, tile_order=0, stream=None):
    """Packed variable-length multi-token update. Returns `out`.

    x is the packed [rows, heads, dim] form, sequence b owning rows
    [cu_seqlens[b], cu_seqlens[b+1]); or the dense [batch, steps, heads, dim]
    form (every operand 4-D), which runs as `batch` regular sequences of `steps`
    rows with no starts tensor. Without cu_seqlens a packed x must have one row
    per sequence."""
    call, result = _packed_call(state, x, dt, A, B, C, cu_seqlens, out, num_accepted_tokens,
                                state_batch_indices, dst_state_batch_indices, D, z, dt_bias,
                                dt_softplus, pad_slot_id, disable_state_update, rand_seed,
                                philox_rounds, steps, heads_per_block, loads_per_lane, tile_order)
    call(stream)
    return result


def prepare_packed_varlen(state, x, dt, A, B, C, cu_seqlens=None, out=None, *,
                          num_accepted_tokens=None, state_batch_indices=None,
                          dst_state_batch_indices=None, D=None, z=None, dt_bias=None,
                          dt_softplus=False, pad_slot_id=-1, disable_state_update=False,
                          rand_seed=None, philox_rounds=10, steps=None, heads_per_block=0,
                          loads_per_lane=0, tile_order=0):
    """`ssu_packed_varlen`'s checks and marshalling, done once; returns a
    PreparedCall whose `out` is the packed (or, for a dense x, the dense) out."""
    call, result = _packed_call(state, x, dt, A, B, C, cu_seqlens, out, num_accepted_tokens,
                                state_batch_indices, dst_state_batch_indices, D, z, dt_bias,
                                dt_softplus, pad_slot_id, disable_state_update, rand_seed,
                                philox_rounds, steps, heads_per_block, loads_per_lane, tile_order,
                                no_copies=True)
    call.out = result
    return call


def _packed_call(state, x, dt, A, B, C, cu_seqlens, out, num_accepted_tokens,
                 state_batch_indices, dst_state_batch_indices, D, z, dt_bias, dt_softplus,
                 pad_slot_id, disable_state_update, rand_seed, philox_rounds, steps,
                 heads_per_block, loads_per_lane, tile_order, no_copies=False):
    """(PreparedCall, the out tensor the public call returns). no_copies: refuse
    dense operands whose flattening would copy them (a prepared call must read
    the caller's tensors, not copies made once)."""
    dense_out = None
    dense_shape = None
    seq_len = 0
    if x.dim() == 4:
        dense_shape = tuple(x.shape)
        batch, dsteps = x.shape[:2]
        rows = batch * dsteps
        if out is not None:
            if not out.is_contiguous() or out.shape != x.shape:
                raise ValueError("a dense out must be contiguous and shaped like x")
            dense_out = out
            out = out.view(rows, *out.shape[2:])
        lead = (batch, dsteps)
        dense = (x, dt, B, C, z)
        dt = _flatten_dense("dt", dt, lead, min_dim=3)
        B, C = _flatten_dense("B", B, lead), _flatten_dense("C", C, lead)
        z = _flatten_dense("z", z, lead)
        x = x.reshape(rows, *x.shape[2:])
        if no_copies and any(a is not None and a.data_ptr() != b.data_ptr()
                             for a, b in zip(dense, (x, dt, B, C, z))):
            raise ValueError("a prepared dense call needs operands that flatten without a copy")
        if cu_seqlens is None:
            seq_len = max(dsteps, 1)
    op, out, rows, _keep = _operands(state, x, dt, A, B, C, out, D, z, dt_bias, dt_softplus,
                                     pad_slot_id, disable_state_update, heads_per_block,
                                     loads_per_lane, tile_order, rand_seed, philox_rounds)
    cu, meta = _index("cu_seqlens", cu_seqlens, state.device)
    na, na_dt = _index("num_accepted_tokens", num_accepted_tokens, state.device)
    if cu is not None:
        if cu.dim() != 1 or cu.shape[0] < 1:
            raise ValueError("cu_seqlens must be a 1-D [sequences + 1] tensor")
        nseq = cu.shape[0] - 1
    elif dense_shape is not None:
        nseq = dense_shape[0]
    else:
        # One row per sequence; count sequences from the per-sequence metadata.
        if na is not None:
            nseq = na.shape[0]
        elif state_batch_indices is not None:
            nseq = state_batch_indices.shape[0]
        elif dst_state_batch_indices is not None:
            nseq = dst_state_batch_indices.shape[0]
        else:
            raise ValueError("a packed call needs cu_seqlens, a dense x, or per-sequence "
                             "metadata (slot tables or num_accepted_tokens)")
        if nseq != rows:
            raise ValueError(f"without cu_seqlens, {rows} rows cannot be split across "
                             f"{nseq} sequences")
        seq_len = 1
    if na is not None and cu is None:
        meta = na_dt
    if na is not None:
        if na.dim() != 1 or na.shape[0] != nseq:
            raise ValueError(f"num_accepted_tokens must be [{nseq}], got {tuple(na.shape)}")
        if cu is not None and na.dtype != cu.dtype:
            raise ValueError("cu_seqlens and num_accepted_tokens must share a dtype")
    src, src_dt, sss, sst, sw = _table("state_batch_indices", state_batch_indices,
                                       state.device, nseq)
    dst, dst_dt, dss, dst_st, dw = _table("dst_state_batch_indices", dst_state_batch_indices,
                                          state.device, nseq)
    if steps is None:
        widths = [w for w in (sw, dw) if w is not None]
        if len(set(widths)) > 1:
            raise ValueError(f"read and write tables have different widths {widths}; pass steps")
        steps = widths[0] if widths else 1
    args = _abi.PackedArgs(
        struct_size=ctypes.sizeof(_abi.PackedArgs), op=op, rows=rows, nseq=nseq,
        cu_seqlens=_ptr(cu), seq_len=seq_len, num_accepted=_ptr(na), meta_dtype=meta,
        src_table=_ptr(src), src_dtype=src_dt, src_seq_stride=sss, src_step_stride=sst,
        dst_table=_ptr(dst), dst_dtype=dst_dt, dst_seq_stride=dss, dst_step_stride=dst_st,
        steps=int(steps))
    if dense_out is not None:
        result = dense_out
    else:
        result = out.view(dense_shape) if dense_shape is not None else out
    keep = (state, x, dt, B, C, z, out, cu, na, src, dst, rand_seed) + _keep
    return PreparedCall("ssu_packed_varlen", args, state.device, out, keep), result


# ------------------------------------------------------------ ring trackers

def _ring_args(ring_start, prev_num_accepted, prev_query_len, state_batch_indices, pad_slot_id):
    trackers = (ring_start, prev_num_accepted, prev_query_len)
    dtypes = {t.dtype for t in trackers}
    if len(dtypes) != 1 or next(iter(dtypes)) not in _INDEX_DTYPES:
        raise ValueError("ring_start, prev_num_accepted and prev_query_len must share an "
                         f"int32 or int64 dtype, got {[t.dtype for t in trackers]}")
    device = ring_start.device
    if device.type != "cuda":
        raise ValueError(f"ring trackers must be on a GPU, got {device}")
    for name, t in zip(("ring_start", "prev_num_accepted", "prev_query_len"), trackers):
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, ring_start on {device}")
        _contig(name, t)
    slots, slot_dt = _index("state_batch_indices", state_batch_indices, device)
    if slots.dim() == 2:
        stride = slots.stride(0)          # the first column of a slot table
    elif slots.dim() == 1:
        stride = slots.stride(0)
    else:
        raise ValueError("state_batch_indices must be [n] or [n, steps]")
    return _abi.RingArgs(
        struct_size=ctypes.sizeof(_abi.RingArgs), ring_start=_ptr(ring_start),
        prev_num_accepted=_ptr(prev_num_accepted), prev_query_len=_ptr(prev_query_len),
        tracker_dtype=_INDEX_DTYPES[ring_start.dtype],
        num_states=min(t.numel() for t in trackers), slots=_ptr(slots), slot_dtype=slot_dt,
        slot_stride=stride, n=slots.shape[0], pad_slot_id=int(pad_slot_id))


@_on_stream
def update_replayssm_ring_trackers(ring_start, prev_num_accepted, prev_query_len,
                                   state_batch_indices, logical_window=None,
                                   ring_buffer_len=None, pad_slot_id=-1, stream=None):
    """Reset the ring trackers of the named slots (logical_window None) or
    advance them by one decoded token. A 2-D slot table names slots by its first
    column. num_states is the shortest tracker's length."""
    lib = library()
    args = _ring_args(ring_start, prev_num_accepted, prev_query_len, state_batch_indices,
                      pad_slot_id)
    if logical_window is None:
        args.reset, args.logical_window, args.ring_buffer_len = 1, 0, 1
    else:
        if ring_buffer_len is None:
            raise ValueError("advancing needs ring_buffer_len")
        args.reset, args.logical_window, args.ring_buffer_len = 0, logical_window, ring_buffer_len
    rc = lib.ssu_ring_update(ctypes.byref(args), _stream(ring_start.device, stream))
    if rc != _abi.SSU_OK:
        _raise(lib, rc, "ssu_ring_update")


@_on_stream
def reset_replayssm_ring_trackers(ring_start, prev_num_accepted, prev_query_len,
                                  state_batch_indices, pad_slot_id=-1, stream=None):
    """Zero the three ring trackers of every named slot."""
    update_replayssm_ring_trackers(ring_start, prev_num_accepted, prev_query_len,
                                   state_batch_indices, pad_slot_id=pad_slot_id, stream=stream)


@_on_stream
def commit_replayssm_ring_trackers(ring_start, prev_num_accepted, prev_query_len,
                                   state_batch_indices, num_accepted_tokens, query_start_loc,
                                   logical_window, ring_buffer_len, pad_slot_id=-1,
                                   stream=None):
    """Settle the previous speculative window of each named slot with the count
    accepted from it, and record the current window's length from query_start_loc."""
    lib = library()
    args = _ring_args(ring_start, prev_num_accepted, prev_query_len, state_batch_indices,
                      pad_slot_id)
    na, na_dt = _index("num_accepted_tokens", num_accepted_tokens, ring_start.device)
    qsl, q_dt = _index("query_start_loc", query_start_loc, ring_start.device)
    if na.dim() != 1 or na.shape[0] < args.n or qsl.dim() != 1 or qsl.shape[0] < args.n + 1:
        raise ValueError("num_accepted_tokens needs n entries and query_start_loc n + 1")
    if na.dtype != qsl.dtype:
        raise ValueError("num_accepted_tokens and query_start_loc must share a dtype")
    args.num_accepted, args.query_start_loc, args.meta_dtype = _ptr(na), _ptr(qsl), na_dt
    args.logical_window, args.ring_buffer_len = logical_window, ring_buffer_len
    rc = lib.ssu_ring_commit(ctypes.byref(args), _stream(ring_start.device, stream))
    if rc != _abi.SSU_OK:
        _raise(lib, rc, "ssu_ring_commit")


# ------------------------------------------------------------------- prefill

# Prefill scratch, one buffer per (device, stream): grown to the largest call
# seen, reused by every later call on that stream (MATE page: the module keeps
# its SSD workspaces across calls, because per-call scratch allocation is what
# makes a wrapper expensive).
_ssd_workspaces = {}


def ssd_workspace_bytes(nchunks, batch, nheads, headdim, dstate, ngroups, chunk_size):
    """Bytes a caller-provided `workspace` of ssd_combined_fwd_varlen must hold:
    the library's figure plus 255 bytes, since the binding aligns the start to 256."""
    return int(library().ssu_ssd_workspace_bytes(nchunks, batch, nheads, headdim, dstate,
                                                 ngroups, chunk_size)) + 255


def _cached_workspace(device, nbytes):
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    with _lock:
        ws = _ssd_workspaces.get(key)
        if ws is None or ws.numel() < nbytes + 255:
            ws = torch.empty(nbytes + 255, dtype=torch.uint8, device=device)
            _ssd_workspaces[key] = ws
        return ws


def reset_ssd_workspaces():
    """Drop every cached prefill workspace (the memory returns to torch's caching
    allocator once no queued kernel uses it)."""
    with _lock:
        _ssd_workspaces.clear()


@_on_stream
def ssd_combined_fwd_varlen(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens,
                            last_chunk_indices, seq_idx, out=None, D=None, z=None,
                            dt_bias=None, dt_softplus=False, dt_limit=(0.0, float("inf")),
                            initial_states=None, return_intermediate_states=False,
                            state_dtype=None, checkpoint_token_indices=None,
                            checkpoint_state_slots=None, checkpoint_states=None, workspace=None,
                            static_scratch=False, stream=None):
    """SSD chunked prefill over packed variable-length requests (include/ssd.h).

    The call and its checks follow `ssd_combined_fwd_varlen` on the MATE page
    "Source code for mate.mamba": x [tokens, heads, dim] and dt [tokens, heads]
    packed over the batch; B, C [tokens, groups, dstate] in x's dtype (fp16 or
    bf16); cu_chunk_seqlens alone maps chunks to tokens, seq_idx[c] names the
    request owning chunk c and decides where each chunk's entering state comes
    from; `out` is written in place when given. Returns every chunk's final state
    [nchunks, heads, dim, dstate] with return_intermediate_states, else each
    request's final state [batch, heads, dim, dstate], in state_dtype (default:
    initial_states' dtype, else C's). The checkpoint_* arguments are refused.

    Scratch: the kernels need a workspace (`ssd_workspace_bytes`). Without
    `workspace` the binding keeps one per (device, stream), grown to the largest
    call seen and reused, so repeated calls allocate only the returned states
    (and `out` when it is not given); calls on one stream are ordered, so they
    can share it. `reset_ssd_workspaces()` frees them. A caller that runs
    prefills concurrently on one stream's behalf, or wants the memory under its
    own control, passes a uint8 tensor of at least `ssd_workspace_bytes(...)`
    bytes as `workspace`. With static_scratch=True the call goes to
    `ssu_ssd_prefill_noalloc`, whose scratch is the library's static per-GPU
    array (SSU_SSD_STATIC_SCRATCH_BYTES; larger calls raise NotImplementedError):
    the binding then allocates only the returned states (and `out` if absent).
    """
    if any(v is not None for v in (checkpoint_token_indices, checkpoint_state_slots,
                                   checkpoint_states)):
        raise NotImplementedError("ssd_combined_fwd_varlen does not support the checkpoint_* "
                                  "arguments")
    if x.dim() != 3 or dt.dim() != 2 or B.dim() != 3 or C.dim() != 3:
        raise ValueError("packed SSD expects x [tokens, heads, dim] and dt [tokens, heads]")
    tokens, heads, dim = x.shape
    groups, dstate = B.shape[1], B.shape[2]
    if dt.shape != (tokens, heads):
        raise ValueError("dt must be [tokens, heads]")
    if B.shape != (tokens, groups, dstate) or C.shape != B.shape:
        raise ValueError("B and C must be [tokens, groups, dstate]")
    if x.dtype not in (torch.float16, torch.bfloat16) or B.dtype != x.dtype or C.dtype != x.dtype:
        raise ValueError("x, B and C must share one of fp16/bf16")
    if dt.dtype not in _IO_DTYPES:
        raise ValueError("dt must be fp32, fp16 or bf16")
    if heads % groups:
        raise ValueError("heads must be divisible by groups")
    if A.shape != (heads,) or A.dtype != torch.float32:
        raise ValueError("A must be fp32 [heads]")
    if dt_bias is not None and (dt_bias.shape != (heads,) or dt_bias.dtype != torch.float32):
        raise ValueError("dt_bias must be fp32 [heads]")
    if chunk_size <= 0:
        raise ValueError("chunk_size must be positive")
    nchunks = cu_chunk_seqlens.numel() - 1
    if nchunks < 1:
        raise ValueError("cu_chunk_seqlens must have at least two entries")
    if seq_idx.numel() != nchunks:
        raise ValueError("seq_idx must hold one request id per logical chunk")
    if cu_seqlens.numel() != last_chunk_indices.numel() + 1:
        raise ValueError("cu_seqlens and last_chunk_indices must describe the same batch")
    batch = last_chunk_indices.numel()
    device = x.device
    if device.type != "cuda":
        raise ValueError(f"x must be on a GPU, got {device}")
    if initial_states is not None:
        if tuple(initial_states.shape[1:]) != (heads, dim, dstate):
            raise ValueError("initial_states must be [batch, heads, dim, dstate]")
        if initial_states.shape[0] != batch:
            raise ValueError("initial_states must hold one row per sequence in cu_seqlens")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x's shape and dtype")
    D_per_dim = 0
    if D is not None:
        if D.shape == (heads, dim):
            D_per_dim = 1
        elif D.shape != (heads,):
            raise ValueError("D must be [heads, dim] or [heads]")
        if D.dtype != torch.float32:
            raise NotImplementedError("D must be fp32")
    if z is not None and z.shape != x.shape:
        raise ValueError("z must match x's shape")
    if z is not None and z.dtype != x.dtype:
        raise ValueError("z must share x's dtype")
    if state_dtype is None:
        state_dtype = initial_states.dtype if initial_states is not None else C.dtype
    if state_dtype not in _STATE_DTYPES:
        raise ValueError("state_dtype must be fp16, bf16 or fp32")
    if initial_states is not None and initial_states.dtype != state_dtype:
        raise NotImplementedError("initial_states must be in state_dtype")
    for name, t in (("x", x), ("dt", dt), ("A", A), ("B", B), ("C", C),
                    ("cu_seqlens", cu_seqlens), ("cu_chunk_seqlens", cu_chunk_seqlens),
                    ("last_chunk_indices", last_chunk_indices), ("seq_idx", seq_idx)):
        if not t.is_contiguous():
            raise ValueError("x, dt, A, B, C and the chunk metadata must be contiguous")
    for name, t in (("out", out), ("z", z), ("D", D), ("dt_bias", dt_bias),
                    ("initial_states", initial_states)):
        _contig(name, t)
    for name, t in (("dt", dt), ("A", A), ("B", B), ("C", C), ("out", out), ("z", z), ("D", D),
                    ("dt_bias", dt_bias), ("initial_states", initial_states),
                    ("cu_chunk_seqlens", cu_chunk_seqlens), ("seq_idx", seq_idx),
                    ("last_chunk_indices", last_chunk_indices)):
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, x is on {device}")
    meta = {cu_chunk_seqlens.dtype, seq_idx.dtype, last_chunk_indices.dtype}
    if len(meta) != 1 or cu_chunk_seqlens.dtype not in _INDEX_DTYPES:
        raise ValueError("cu_chunk_seqlens, seq_idx and last_chunk_indices must share int32 or "
                         "int64")
    lib = library()
    rows = nchunks if return_intermediate_states else batch
    states = torch.empty((rows, heads, dim, dstate), dtype=state_dtype, device=device)
    ws_bytes = lib.ssu_ssd_workspace_bytes(nchunks, batch, heads, dim, dstate, groups,
                                           int(chunk_size))
    if static_scratch:
        if workspace is not None:
            raise ValueError("static_scratch and workspace exclude each other")
        ws_ptr, ws_bytes = None, 0
    else:
        if workspace is None:
            workspace = _cached_workspace(device, ws_bytes)
        elif (workspace.device != device or workspace.dtype != torch.uint8 or
              not workspace.is_contiguous() or workspace.numel() < ws_bytes + 255):
            raise ValueError(f"workspace must be a contiguous uint8 tensor on {device} of at "
                             f"least ssd_workspace_bytes(...) = {ws_bytes + 255} bytes")
        ws_ptr = (workspace.data_ptr() + 255) // 256 * 256
    args = _abi.SsdArgs()
    args.struct_size = ctypes.sizeof(_abi.SsdArgs)
    args.tokens, args.nheads, args.headdim, args.dstate, args.ngroups = (tokens, heads, dim,
                                                                         dstate, groups)
    args.chunk_size, args.nchunks, args.batch = int(chunk_size), nchunks, batch
    args.x, args.dt, args.A, args.B, args.C = _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C)
    args.D, args.z, args.dt_bias = _ptr(D), _ptr(z), _ptr(dt_bias)
    args.io_dtype, args.dt_dtype = _IO_DTYPES[x.dtype], _IO_DTYPES[dt.dtype]
    args.D_per_dim, args.dt_softplus = D_per_dim, int(bool(dt_softplus))
    args.dt_min, args.dt_max = float(dt_limit[0]), float(dt_limit[1])
    args.cu_chunk_seqlens, args.seq_idx = _ptr(cu_chunk_seqlens), _ptr(seq_idx)
    args.last_chunk_indices = _ptr(last_chunk_indices)
    args.meta_dtype = _INDEX_DTYPES[cu_chunk_seqlens.dtype]
    args.state_dtype = _STATE_DTYPES[state_dtype]
    args.initial_states, args.out, args.states = _ptr(initial_states), _ptr(out), _ptr(states)
    args.return_intermediate_states = int(bool(return_intermediate_states))
    args.workspace, args.workspace_bytes = ws_ptr, ws_bytes
    entry = lib.ssu_ssd_prefill_noalloc if static_scratch else lib.ssu_ssd_prefill
    rc = entry(ctypes.byref(args), _stream(device, stream))
    if rc != _abi.SSU_OK:
        _raise(lib, rc, entry.__name__)
    return states
