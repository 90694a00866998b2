"""Seeded synthetic decode workloads for the selective state update.

This module only draws inputs: shapes, value distributions and slot structure.
It holds none of the update's arithmetic, so the GPU path and the CPU reference
can both consume what it produces without sharing any of the method.

Every tensor is drawn from its own torch generator, seeded from (workload seed,
tensor name), on the device it is asked for; the slot structure (permutations,
pads, lengths, acceptance counts) is drawn on the CPU, so it is the same on every
device. Low-precision operands are drawn in
fp32 and rounded to nearest-even by the dtype cast, so both sides of a comparison
see identical bits. Values differ between devices (CPU and GPU generators are
different streams); a comparison always hands the same tensors to both sides.

Named workloads (one GPU each, at their real decode shapes):
  tiny        batch 4, 8 heads x 64 x dstate 16, 1 group, everything fp32,
              identity slots, no gate, no pads.
  mamba2_2p7b batch 256, 80 heads x 64 x 128, 1 group; fp32 state in 512 slots,
              read slots a random subset of the cache, written in place; bf16
              x/B/C/z; softplus and gate on.
  bf16_state  batch 1024, 64 heads x 64 x 128, 8 groups; bf16 state in 2048
              slots; ~10 % of read slots are the pad id -1; every sequence writes
              a distinct slot that no sequence reads; fp16 x/B/C; no gate.
  nemotron_h  batch 512, 128 heads x 64 x 128, 8 groups; fp32 state in 1024
              slots, in place; bf16 x/B/C/z; dt ~ U(-4, 0), A = -exp(U(0, 3)).
              Also run with the state update disabled (read-only).
  packed_mtp  256 sequences of 1..4 speculative tokens packed by int32
              cu_seqlens; 80 heads x 64 x 128, 1 group; fp32 state in 2048 slots;
              a [256, 4] table of distinct slots serves as both the read and the
              write table; the acceptance count ~ U{1..len} picks the read entry;
              5 % of sequences have an all-pad table row.
  dense_mtp   the Mamba2-2.7B shape in the dense [256, 2, ...] layout (one draft
              token per sequence), slot table [256, 2] of 1024 slots, 5 % pads.
  bf16_state_sr  bf16_state with stochastic rounding of the stored states.

SSD prefill workloads (`SSD_NAMED`, packed prompts cut into chunks):
  ssd_mamba2_2p7b  16 prompts of U{256..2048} tokens, 80 heads x 64 x 128,
                   1 group, chunk 256; bf16 x/B/C/z, fp32 states, fresh prompts
                   (no initial states).
  ssd_nemotron_h   8 prompts of U{512..4096} tokens, 128 heads x 64 x 128,
                   8 groups, chunk 128; bf16 io, fp32 states continuing from
                   initial states; dt ~ U(-4, 0), A = -exp(U(0, 3)).
  ssd_small        prompts of 1, 255, 256, 257, 700 and 37 tokens, 4 heads x 64
                   x 128, 2 groups, chunk 256; initial states.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_INDEX_DTYPES = {"i32": torch.int32, "i64": torch.int64}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name] if name in _TORCH_DTYPES else _INDEX_DTYPES[name]


def _generator(seed: int, name: str, device) -> torch.Generator:
    digest = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(digest[:8], "little") & ((1 << 63) - 1))
    return g


def normal(shape, seed, name, device, dtype=torch.float32):
    t = torch.randn(shape, generator=_generator(seed, name, device), device=device,
                    dtype=torch.float32)
    return t.to(dtype)


def uniform(shape, lo, hi, seed, name, device):
    t = torch.rand(shape, generator=_generator(seed, name, device), device=device,
                   dtype=torch.float32)
    return t * (hi - lo) + lo


def permutation(n, seed, name, device):
    """A seeded permutation of range(n), drawn on the CPU whatever the device, so
    that the slot structure (which slots, which pads) of a workload is the same
    on every device and its byte accounting can be done on either."""
    return torch.randperm(n, generator=_generator(seed, name, "cpu")).to(device)


@dataclass
class Workload:
    """One call's operands. `mode` is "one_token" or "packed"."""
    name: str
    mode: str
    state: torch.Tensor                    # [nslots, H, P, N]
    x: torch.Tensor                        # [rows, H, P]
    dt: torch.Tensor                       # [rows, H] or [rows, H, P], fp32
    A: torch.Tensor                        # [H] fp32
    B: torch.Tensor                        # [rows, G, N]
    C: torch.Tensor                        # [rows, G, N]
    D: Optional[torch.Tensor] = None       # [H] fp32
    z: Optional[torch.Tensor] = None       # [rows, H, P]
    dt_bias: Optional[torch.Tensor] = None  # [H] fp32
    rand_seed: Optional[torch.Tensor] = None  # [1] int64: stochastic rounding of 16-bit state
    philox_rounds: int = 10
    dt_softplus: bool = True
    pad_slot_id: int = -1
    disable_state_update: bool = False
    # one-token slot vectors [batch]
    src: Optional[torch.Tensor] = None
    dst: Optional[torch.Tensor] = None
    # packed metadata
    cu_seqlens: Optional[torch.Tensor] = None      # [nseq + 1]
    num_accepted: Optional[torch.Tensor] = None    # [nseq]
    src_table: Optional[torch.Tensor] = None       # [nseq, steps]
    dst_table: Optional[torch.Tensor] = None       # [nseq, steps]
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def dims(self):
        nslots, H, P, N = self.state.shape
        return nslots, H, P, N, self.B.shape[1]

    def out_sentinel(self) -> torch.Tensor:
        """An `out` buffer pre-filled with NaN, so rows the call must not write stay
        recognisable bit for bit."""
        return torch.full(self.x.shape, float("nan"), dtype=self.x.dtype,
                          device=self.x.device)

    def to(self, device) -> "Workload":
        kw = {}
        for k, v in self.__dict__.items():
            kw[k] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


def operands(seed, rows, H, P, N, G, *, device, io="bf16", with_z=True,
             with_D=True, with_bias=True, dt_range=(-3.0, 0.0), a_log_range=(0.0, 2.0),
             dt_per_dim=False):
    """x/B/C/z ~ N(0,1) in the io dtype; dt ~ U(dt_range) fp32; dt_bias ~ U(-1,1);
    A = -exp(U(a_log_range)); D ~ N(0,1). A, D, dt_bias are one value per head."""
    iod = torch_dtype(io)
    dt_shape = (rows, H, P) if dt_per_dim else (rows, H)
    return dict(
        x=normal((rows, H, P), seed, "x", device, iod),
        dt=uniform(dt_shape, dt_range[0], dt_range[1], seed, "dt", device),
        A=-torch.exp(uniform((H,), a_log_range[0], a_log_range[1], seed, "A", device)),
        B=normal((rows, G, N), seed, "B", device, iod),
        C=normal((rows, G, N), seed, "C", device, iod),
        D=normal((H,), seed, "D", device) if with_D else None,
        z=normal((rows, H, P), seed, "z", device, iod) if with_z else None,
        dt_bias=uniform((H,), -1.0, 1.0, seed, "dt_bias", device) if with_bias else None,
    )


def state_cache(seed, nslots, H, P, N, *, device, dtype="f32"):
    """The slot cache, ~N(0,1). A draw of exactly +-0 has probability ~0, and the
    copy-placement checks rely on non-zero state values."""
    s = normal((nslots, H, P, N), seed, "state", device, torch_dtype(dtype))
    return s.masked_fill(s == 0, 0.5)


def one_token(name, seed, *, batch, H, P, N, G, nslots, device, state_dtype="f32",
              io="bf16", with_z=True, pad_fraction=0.0, dst_mode="same",
              index_dtype="i32", identity=False, **kw) -> Workload:
    """A one-token decode batch.

    identity: no slot vectors (sequence b uses slot b).
    Otherwise src = first `batch` entries of a random permutation of the slots,
    with round(pad_fraction * batch) random positions set to -1; dst_mode "same"
    passes dst = src, "distinct" the next `batch` entries of the permutation
    (disjoint from every src), "none" passes no dst vector."""
    ops = operands(seed, batch, H, P, N, G, device=device, io=io, with_z=with_z, **kw)
    state = state_cache(seed, nslots, H, P, N, device=device, dtype=state_dtype)
    src = dst = None
    if not identity:
        perm = permutation(nslots, seed, "slots", device)
        idt = torch_dtype(index_dtype)
        src = perm[:batch].to(idt).clone()
        npad = int(round(pad_fraction * batch))
        if npad:
            where = permutation(batch, seed, "pads", device)[:npad]
            src[where] = -1
        if dst_mode == "same":
            dst = src.clone()
        elif dst_mode == "distinct":
            if nslots < 2 * batch:
                raise ValueError("distinct destinations need nslots >= 2 * batch")
            dst = perm[batch:2 * batch].to(idt).clone()
        elif dst_mode != "none":
            raise ValueError(dst_mode)
    return Workload(name=name, mode="one_token", state=state, src=src, dst=dst,
                    meta=dict(seed=seed, state_dtype=state_dtype, io=io), **ops)


def packed(name, seed, *, nseq, max_len, H, P, N, G, nslots, device, state_dtype="f32",
           io="bf16", with_z=True, pad_fraction=0.0, meta_dtype="i32",
           index_dtype="i32", lengths=None, accepted=True, dense=False, **kw) -> Workload:
    """A packed MTP batch: lengths ~ U{1..max_len} (or given), a [nseq, max_len]
    table of distinct slots used as both read and write table, acceptance counts
    ~ U{1..len}, and round(pad_fraction * nseq) sequences whose table row is all
    pad (-1). dense=True: every sequence has max_len rows and the call is meant to
    be made in the dense [nseq, max_len, ...] layout (meta["dense"])."""
    if dense:
        lengths = [max_len] * nseq
    if lengths is None:
        lengths = torch.randint(1, max_len + 1, (nseq,),
                                generator=_generator(seed, "lengths", "cpu"))
    lengths = torch.as_tensor(lengths, dtype=torch.int64).cpu()
    rows = int(lengths.sum())
    cu = torch.zeros(nseq + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    mdt = torch_dtype(meta_dtype)
    ops = operands(seed, rows, H, P, N, G, device=device, io=io, with_z=with_z, **kw)
    state = state_cache(seed, nslots, H, P, N, device=device, dtype=state_dtype)
    if nslots < nseq * max_len:
        raise ValueError("the slot table needs nslots >= nseq * max_len")
    perm = permutation(nslots, seed, "slots", device)
    table = perm[:nseq * max_len].reshape(nseq, max_len).to(torch_dtype(index_dtype))
    npad = int(round(pad_fraction * nseq))
    if npad:
        where = permutation(nseq, seed, "pads", device)[:npad]
        table[where] = -1
    num_acc = None
    if accepted:
        u = torch.rand((nseq,), generator=_generator(seed, "accepted", "cpu"))
        k = torch.clamp((u * lengths.clamp(min=1)).floor().to(torch.int64) + 1,
                        max=max_len)
        num_acc = k.to(mdt).to(device)
    return Workload(name=name, mode="packed", state=state, cu_seqlens=cu.to(mdt).to(device),
                    num_accepted=num_acc, src_table=table, dst_table=table,
                    meta=dict(seed=seed, state_dtype=state_dtype, io=io,
                              lengths=lengths.tolist(), dense=dense), **ops)


# The five named decode workloads. `seed` defaults to the workload's ordinal.
def tiny(device, seed=0):
    return one_token("tiny", seed, batch=4, H=8, P=64, N=16, G=1, nslots=4,
                     device=device, state_dtype="f32", io="f32", with_z=False,
                     identity=True)


def mamba2_2p7b(device, seed=1):
    return one_token("mamba2_2p7b", seed, batch=256, H=80, P=64, N=128, G=1, nslots=512,
                     device=device, state_dtype="f32", io="bf16", with_z=True,
                     dst_mode="same")


def bf16_state(device, seed=2):
    return one_token("bf16_state", seed, batch=1024, H=64, P=64, N=128, G=8, nslots=2048,
                     device=device, state_dtype="bf16", io="f16", with_z=False,
                     pad_fraction=0.1, dst_mode="distinct")


def nemotron_h(device, seed=3, disable_state_update=False):
    w = one_token("nemotron_h", seed, batch=512, H=128, P=64, N=128, G=8, nslots=1024,
                  device=device, state_dtype="f32", io="bf16", with_z=True,
                  dst_mode="same", dt_range=(-4.0, 0.0), a_log_range=(0.0, 3.0))
    if disable_state_update:
        w.name = "nemotron_h_readonly"
        w.disable_state_update = True
    return w


def dense_mtp(device, seed=5):
    """Mamba2-2.7B-shaped MTP decode in the dense [batch, steps] layout: 256
    sequences of 2 tokens (one draft), no starts tensor."""
    return packed("dense_mtp", seed, nseq=256, max_len=2, H=80, P=64, N=128, G=1,
                  nslots=1024, device=device, state_dtype="f32", io="bf16",
                  with_z=True, pad_fraction=0.05, dense=True)


def bf16_state_sr(device, seed=2):
    """bf16_state with stochastic rounding of the stored states (seeded Philox)."""
    w = bf16_state(device, seed)
    w.name = "bf16_state_sr"
    w.rand_seed = torch.tensor([0x5EED_0000_2B16 + seed], dtype=torch.int64, device=device)
    return w


def packed_mtp(device, seed=4):
    return packed("packed_mtp", seed, nseq=256, max_len=4, H=80, P=64, N=128, G=1,
                  nslots=2048, device=device, state_dtype="f32", io="bf16",
                  with_z=True, pad_fraction=0.05)


@dataclass
class SsdWorkload:
    """One SSD prefill call's operands and chunk metadata (int tensors on the
    workload's device)."""
    name: str
    x: torch.Tensor                    # [tokens, H, P] io
    dt: torch.Tensor                   # [tokens, H]
    A: torch.Tensor                    # [H] fp32
    B: torch.Tensor                    # [tokens, G, N] io
    C: torch.Tensor                    # [tokens, G, N] io
    chunk_size: int
    cu_seqlens: torch.Tensor           # [batch + 1]
    cu_chunk_seqlens: torch.Tensor     # [nchunks + 1]
    seq_idx: torch.Tensor              # [nchunks]
    last_chunk_indices: torch.Tensor   # [batch]
    state_dtype: torch.dtype
    D: Optional[torch.Tensor] = None   # [H] or [H, P] fp32
    z: Optional[torch.Tensor] = None
    dt_bias: Optional[torch.Tensor] = None
    initial_states: Optional[torch.Tensor] = None  # [batch, H, P, N] state dtype
    dt_softplus: bool = True
    dt_limit: tuple = (0.0, float("inf"))
    return_intermediate_states: bool = False
    meta: dict = field(default_factory=dict)

    def kwargs(self) -> dict:
        """Keyword arguments of `ssd_combined_fwd_varlen` for this call."""
        return dict(D=self.D, z=self.z, dt_bias=self.dt_bias, dt_softplus=self.dt_softplus,
                    dt_limit=self.dt_limit, initial_states=self.initial_states,
                    return_intermediate_states=self.return_intermediate_states,
                    state_dtype=self.state_dtype)

    def args(self) -> tuple:
        return (self.x, self.dt, self.A, self.B, self.C, self.chunk_size, self.cu_seqlens,
                self.cu_chunk_seqlens, self.last_chunk_indices, self.seq_idx)


def chunk_metadata(lengths, chunk_size, request_ids=None):
    """Cut packed requests into chunks of chunk_size tokens (a request's last
    chunk may be shorter): cu_seqlens, cu_chunk_seqlens, seq_idx (the request id
    of each chunk; 0, 1, ... unless given) and last_chunk_indices, as lists."""
    ids = list(range(len(lengths))) if request_ids is None else list(request_ids)
    cu, cc, seq_idx, last = [0], [0], [], []
    for b, L in enumerate(lengths):
        cu.append(cu[-1] + L)
        pos = 0
        while True:
            step = min(chunk_size, L - pos)
            cc.append(cc[-1] + step)
            seq_idx.append(ids[b])
            pos += step
            if pos >= L:
                break
        last.append(len(seq_idx) - 1)
    return cu, cc, seq_idx, last


def ssd(name, seed, *, lengths, H, P, N, G, chunk, device, io="bf16", state_dtype="f32",
        dt_dtype="f32", with_init=False, with_z=True, D_per_dim=False, dt_range=(-3.0, 0.0),
        a_log_range=(0.0, 2.0), meta_dtype="i32", request_ids=None, **kw) -> SsdWorkload:
    """A packed prefill: x/B/C/z ~ N(0,1) in the io dtype, dt ~ U(dt_range),
    dt_bias ~ U(-1, 1), A = -exp(U(a_log_range)), D ~ N(0, 1), initial states
    ~ N(0, 1) in the state dtype."""
    lengths = [int(v) for v in lengths]
    tokens = sum(lengths)
    ops = operands(seed, tokens, H, P, N, G, device=device, io=io, with_z=with_z,
                   dt_range=dt_range, a_log_range=a_log_range)
    ops["dt"] = ops["dt"].to(torch_dtype(dt_dtype))
    if D_per_dim:
        ops["D"] = normal((H, P), seed, "D2", device)
    cu, cc, seq_idx, last = chunk_metadata(lengths, chunk, request_ids)
    mdt = torch_dtype(meta_dtype)
    t = lambda v: torch.tensor(v, dtype=mdt, device=device)
    batch = len(last)
    init = None
    if with_init:
        init = normal((batch, H, P, N), seed, "initial_states", device, torch_dtype(state_dtype))
    return SsdWorkload(name=name, chunk_size=chunk, cu_seqlens=t(cu), cu_chunk_seqlens=t(cc),
                       seq_idx=t(seq_idx), last_chunk_indices=t(last),
                       state_dtype=torch_dtype(state_dtype), initial_states=init,
                       meta=dict(seed=seed, lengths=lengths, io=io), **ops, **kw)


def _lengths(n, lo, hi, seed):
    g = _generator(seed, "lengths", "cpu")
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def ssd_mamba2_2p7b(device, seed=11):
    return ssd("ssd_mamba2_2p7b", seed, lengths=_lengths(16, 256, 2048, seed), H=80, P=64,
               N=128, G=1, chunk=256, device=device)


def ssd_nemotron_h(device, seed=12):
    return ssd("ssd_nemotron_h", seed, lengths=_lengths(8, 512, 4096, seed), H=128, P=64,
               N=128, G=8, chunk=128, device=device, with_init=True, dt_range=(-4.0, 0.0),
               a_log_range=(0.0, 3.0))


def ssd_small(device, seed=13):
    return ssd("ssd_small", seed, lengths=[1, 255, 256, 257, 700, 37], H=4, P=64, N=128, G=2,
               chunk=256, device=device, with_init=True)


SSD_NAMED = {
    "ssd_mamba2_2p7b": ssd_mamba2_2p7b,
    "ssd_nemotron_h": ssd_nemotron_h,
    "ssd_small": ssd_small,
}


NAMED = {
    "tiny": tiny,
    "mamba2_2p7b": mamba2_2p7b,
    "bf16_state": bf16_state,
    "nemotron_h": nemotron_h,
    "nemotron_h_readonly": lambda device, seed=3: nemotron_h(device, seed, True),
    "packed_mtp": packed_mtp,
    "dense_mtp": dense_mtp,
    "bf16_state_sr": bf16_state_sr,
}
