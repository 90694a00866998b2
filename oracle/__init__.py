"""Plain fp64 CPU reference of the Mamba-2 selective state update (SSU).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library never
calls it, and it shares no code with the GPU library.

The arithmetic lives in ``ssu_oracle.c`` (plain C, fp64, loops in the order
sequence -> head -> row -> dstate): the decode-time selective state update, the
ReplaySSM ring trackers, Philox4x32 and stochastic rounding, and the SSD chunked
prefill as the token-by-token recurrence it equals. This module only compiles it with gcc, loads
it with ctypes and widens operands: every fp16/bf16/fp32 value is exactly
representable in fp64, so the widening loses nothing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssu_oracle.c")
LIBRARY = os.path.join(HERE, "libssu_oracle.so")

# Plain ISO C: no fused multiply-add contraction, no fast-math.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle C source into a shared library and return its path."""
    tmp = output + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, output)
    return output


class _Rounding(ctypes.Structure):
    _fields_ = [("sr_format", ctypes.c_int), ("rand_seed", ctypes.c_uint64),
                ("philox_rounds", ctypes.c_int), ("row_base", ctypes.c_int64)]


SR_FORMATS = {None: 0, "f16": 1, "bf16": 2}

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _idx(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _p(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


@dataclass
class Result:
    out: np.ndarray        # [rows, nheads, headdim] fp64; rows of inert sequences keep out_init
    state: np.ndarray      # [nslots, nheads, headdim, dstate] fp64 after the call


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_ssu_one_token.restype = _int
        _rp = ctypes.POINTER(_Rounding)
        lib.oracle_ssu_one_token.argtypes = [
            _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64,
            _dp, _dp, _int, _dp, _dp, _dp, _dp, _dp, _dp, _int,
            _ip, _ip, _i64, _int, _rp, _dp]
        lib.oracle_ssu_packed_varlen.restype = _int
        lib.oracle_ssu_packed_varlen.argtypes = [
            _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
            _ip, _ip, _ip, _i64, _i64, _ip, _i64, _i64, _i64,
            _dp, _dp, _int, _dp, _dp, _dp, _dp, _dp, _dp, _int,
            _i64, _int, _rp, _dp]
        _u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32.restype = None
        lib.oracle_philox4x32.argtypes = [_u32p, _u32p, _int, _u32p]
        lib.oracle_round_stochastic.restype = None
        lib.oracle_round_stochastic.argtypes = [_dp, _u32p, _i64, _int, _dp]
        for f in (lib.oracle_ring_update, lib.oracle_ring_commit):
            f.restype = _int
        lib.oracle_ring_update.argtypes = [_ip, _ip, _ip, _i64, _ip, _i64, _i64, _int, _i64,
                                           _i64, _i64]
        lib.oracle_ring_commit.argtypes = [_ip, _ip, _ip, _i64, _ip, _i64, _i64, _ip, _ip,
                                           _i64, _i64, _i64]
        _d = ctypes.c_double
        lib.oracle_ssd_prefill.restype = _int
        lib.oracle_ssd_prefill.argtypes = [
            _i64, _i64, _i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp, _int, _dp, _dp, _int,
            _d, _d, _i64, _i64, _ip, _ip, _i64, _ip, _dp, _dp, _dp, _dp]
        self.lib = lib

    @staticmethod
    def _common(state, x, dt, A, B, C, D, z, dt_bias, out_init):
        state = _f64(state)
        if state.ndim != 4:
            raise ValueError("state must be [nslots, nheads, headdim, dstate]")
        x = _f64(x)
        dt = _f64(dt)
        rows = x.shape[0]
        if dt.ndim == 3 and dt.shape[2] == 1:
            dt = np.ascontiguousarray(dt[:, :, 0])
        dt_per_dim = 1 if dt.ndim == 3 else 0
        if out_init is None:
            out = np.full(x.shape, np.nan, dtype=np.float64)
        else:
            out = _f64(out_init).copy()
        return (state, x, dt, dt_per_dim, _f64(A), _f64(B), _f64(C), _f64(D),
                _f64(z), _f64(dt_bias), out, rows)

    @staticmethod
    def _rounding(sr_format, rand_seed, philox_rounds, row_base=0):
        if sr_format is None:
            return None
        return ctypes.byref(_Rounding(SR_FORMATS[sr_format], int(rand_seed) & (2**64 - 1),
                                      int(philox_rounds), int(row_base)))

    def philox4x32(self, counter, key, rounds=10):
        """The four output words of Philox4x32 for one counter and key."""
        c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in counter])
        k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
        o = (ctypes.c_uint32 * 4)()
        self.lib.oracle_philox4x32(c, k, int(rounds), o)
        return list(o)

    def round_stochastic(self, v, words, fmt):
        """SR of each v[i] to fmt ("f16" or "bf16") with random word words[i]."""
        v = _f64(v).reshape(-1)
        w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32).reshape(-1))
        assert v.shape == w.shape
        out = np.empty_like(v)
        self.lib.oracle_round_stochastic(_p(v, _dp), w.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                         v.shape[0], SR_FORMATS[fmt], _p(out, _dp))
        return out

    def one_token(self, state, x, dt, A, B, C, *, D=None, z=None, dt_bias=None,
                  dt_softplus=False, src=None, dst=None, pad_slot_id=-1,
                  disable_state_update=False, out_init=None, sr_format=None, rand_seed=0,
                  philox_rounds=10, sr_row_base=0) -> Result:
        """One token per sequence: row b of x/dt/B/C/z/out is sequence b.
        sr_row_base: the call-wide row number of row 0, for the stochastic
        rounding's counters when this problem is cut out of a larger call."""
        (state, x, dt, dt_per_dim, A, B, C, D, z, dt_bias, out,
         batch) = self._common(state, x, dt, A, B, C, D, z, dt_bias, out_init)
        nslots, H, P, N = state.shape
        G = B.shape[1]
        src, dst = _idx(src), _idx(dst)
        state_out = np.empty_like(state)
        rc = self.lib.oracle_ssu_one_token(
            _p(state, _dp), _p(state_out, _dp), nslots, H, P, N, G, batch,
            _p(x, _dp), _p(dt, _dp), dt_per_dim, _p(A, _dp), _p(B, _dp), _p(C, _dp),
            _p(D, _dp), _p(z, _dp), _p(dt_bias, _dp), int(bool(dt_softplus)),
            _p(src, _ip), _p(dst, _ip), int(pad_slot_id), int(bool(disable_state_update)),
            self._rounding(sr_format, rand_seed, philox_rounds, sr_row_base), _p(out, _dp))
        if rc != 0:
            raise ValueError("oracle_ssu_one_token rejected its arguments")
        return Result(out, state_out)

    def packed_varlen(self, state, x, dt, A, B, C, cu_seqlens, *, num_accepted=None,
                      src_table=None, src_strides=None, dst_table=None, dst_strides=None,
                      steps=None, D=None, z=None, dt_bias=None, dt_softplus=False,
                      pad_slot_id=-1, disable_state_update=False, out_init=None,
                      sr_format=None, rand_seed=0, philox_rounds=10, sr_row_base=0) -> Result:
        """Packed varlen form. A 2-D table [nseq, steps] takes strides (steps, 1)
        unless strides are given; a flat table needs explicit strides and steps."""
        (state, x, dt, dt_per_dim, A, B, C, D, z, dt_bias, out,
         rows) = self._common(state, x, dt, A, B, C, D, z, dt_bias, out_init)
        nslots, H, P, N = state.shape
        G = B.shape[1]
        cu = _idx(cu_seqlens)
        nseq = cu.shape[0] - 1
        na = _idx(num_accepted)

        def table(t, strides):
            if t is None:
                return None, 0, 0, None
            t = _idx(t)
            if strides is None:
                if t.ndim != 2:
                    raise ValueError("a flat table needs explicit strides")
                strides = (t.shape[1], 1)
            width = t.shape[1] if t.ndim == 2 else None
            return t.reshape(-1), int(strides[0]), int(strides[1]), width

        st, sss, sst, sw = table(src_table, src_strides)
        dtb, dss, dst_, dw = table(dst_table, dst_strides)
        if steps is None:
            steps = sw if sw is not None else (dw if dw is not None else 1)
        state_out = np.empty_like(state)
        rc = self.lib.oracle_ssu_packed_varlen(
            _p(state, _dp), _p(state_out, _dp), nslots, H, P, N, G, rows, nseq,
            _p(cu, _ip), _p(na, _ip), _p(st, _ip), sss, sst, _p(dtb, _ip), dss, dst_,
            int(steps), _p(x, _dp), _p(dt, _dp), dt_per_dim, _p(A, _dp), _p(B, _dp),
            _p(C, _dp), _p(D, _dp), _p(z, _dp), _p(dt_bias, _dp), int(bool(dt_softplus)),
            int(pad_slot_id), int(bool(disable_state_update)),
            self._rounding(sr_format, rand_seed, philox_rounds, sr_row_base), _p(out, _dp))
        if rc != 0:
            raise ValueError("oracle_ssu_packed_varlen rejected its arguments")
        return Result(out, state_out)


@dataclass
class Rings:
    ring_start: np.ndarray
    prev_num_accepted: np.ndarray
    prev_query_len: np.ndarray


def _rings(ring_start, prev_num_accepted, prev_query_len):
    return Rings(*(_idx(a).copy() for a in (ring_start, prev_num_accepted, prev_query_len)))


def _ring_slots(slots, slot_stride):
    s = _idx(slots).reshape(-1)
    if slot_stride is None:
        slot_stride = 1
    n = (s.shape[0] - 1) // slot_stride + 1 if s.shape[0] else 0
    return s, int(slot_stride), n


def _ring_update(self, ring_start, prev_num_accepted, prev_query_len, slots, *,
                 logical_window=None, ring_buffer_len=None, pad_slot_id=-1,
                 slot_stride=None, n=None) -> Rings:
    """Reset (logical_window None) or advance the trackers of the named slots.
    Returns updated copies; num_states is the shortest tracker's length."""
    r = _rings(ring_start, prev_num_accepted, prev_query_len)
    s, stride, n_all = _ring_slots(slots, slot_stride)
    n = n_all if n is None else n
    num_states = min(a.shape[0] for a in (r.ring_start, r.prev_num_accepted, r.prev_query_len))
    reset = logical_window is None
    rc = self.lib.oracle_ring_update(
        _p(r.ring_start, _ip), _p(r.prev_num_accepted, _ip), _p(r.prev_query_len, _ip),
        num_states, _p(s, _ip), stride, n, int(reset), 0 if reset else int(logical_window),
        1 if reset else int(ring_buffer_len), int(pad_slot_id))
    if rc != 0:
        raise ValueError("oracle_ring_update rejected its arguments")
    return r


def _ring_commit(self, ring_start, prev_num_accepted, prev_query_len, slots, num_accepted,
                 query_start_loc, *, logical_window, ring_buffer_len, pad_slot_id=-1,
                 slot_stride=None, n=None) -> Rings:
    r = _rings(ring_start, prev_num_accepted, prev_query_len)
    s, stride, n_all = _ring_slots(slots, slot_stride)
    n = n_all if n is None else n
    num_states = min(a.shape[0] for a in (r.ring_start, r.prev_num_accepted, r.prev_query_len))
    na, qsl = _idx(num_accepted), _idx(query_start_loc)
    rc = self.lib.oracle_ring_commit(
        _p(r.ring_start, _ip), _p(r.prev_num_accepted, _ip), _p(r.prev_query_len, _ip),
        num_states, _p(s, _ip), stride, n, _p(na, _ip), _p(qsl, _ip), int(logical_window),
        int(ring_buffer_len), int(pad_slot_id))
    if rc != 0:
        raise ValueError("oracle_ring_commit rejected its arguments")
    return r


Oracle.ring_update = _ring_update
Oracle.ring_commit = _ring_commit


@dataclass
class SsdResult:
    out: np.ndarray            # [tokens, nheads, headdim]; rows no chunk covers keep out_init
    chunk_states: np.ndarray   # [nchunks, nheads, headdim, dstate]: state after each chunk
    final_states: np.ndarray   # [batch, nheads, headdim, dstate]: chunk_states[last_chunk_indices]


def _ssd_prefill(self, x, dt, A, B, C, chunk_size, cu_chunk_seqlens, seq_idx,
                 last_chunk_indices, *, D=None, z=None, dt_bias=None, dt_softplus=False,
                 dt_limit=(0.0, float("inf")), initial_states=None,
                 out_init=None) -> SsdResult:
    """SSD chunked prefill over packed tokens (x [tokens, heads, dim], dt
    [tokens, heads], B/C [tokens, groups, dstate]). D is [heads] or [heads, dim]."""
    x, dt, A, B, C = (_f64(a) for a in (x, dt, A, B, C))
    D, z, dt_bias, init = (_f64(a) for a in (D, z, dt_bias, initial_states))
    tokens, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cc, si, lci = _idx(cu_chunk_seqlens), _idx(seq_idx), _idx(last_chunk_indices)
    nchunks, batch = cc.shape[0] - 1, lci.shape[0]
    D_per_dim = 1 if D is not None and D.ndim == 2 else 0
    out = np.full(x.shape, np.nan) if out_init is None else _f64(out_init).copy()
    chunk_states = np.empty((nchunks, H, P, N))
    final_states = np.empty((batch, H, P, N))
    rc = self.lib.oracle_ssd_prefill(
        tokens, H, P, N, G, _p(x, _dp), _p(dt, _dp), _p(A, _dp), _p(B, _dp), _p(C, _dp),
        _p(D, _dp), D_per_dim, _p(z, _dp), _p(dt_bias, _dp), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), int(chunk_size), nchunks, _p(cc, _ip),
        _p(si, _ip), batch, _p(lci, _ip), _p(init, _dp), _p(out, _dp),
        _p(chunk_states, _dp), _p(final_states, _dp))
    if rc != 0:
        raise ValueError("oracle_ssd_prefill rejected its arguments")
    return SsdResult(out, chunk_states, final_states)


Oracle.ssd_prefill = _ssd_prefill


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``ssu_oracle.c``; compiled on first use if absent."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
