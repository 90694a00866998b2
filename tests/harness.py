"""Run the GPU path and the fp64 oracle on the same inputs and compare them.

Test infrastructure: the GPU side goes through the Python binding (and so the
C ABI); the oracle side widens the very same tensors to fp64 on the CPU. For
full-size workloads the oracle runs on runs of consecutive sequences that
together cover the whole call: each run's rows and the slots it touches are cut
out, slot ids renumbered, and the oracle's results compared with the matching
rows and slots of the full GPU run.

Tolerances (per compared tensor):
  fp32 results   max |gpu - ref| <= 1e-5 * max(1, max |ref|)
  fp16 / bf16    |gpu - ref| <= 1e-2 + 2e-2 |ref| element-wise
Placement (which slots change, which out rows are written) is compared exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import selective_state_update_ssu_amd as ssu
from selective_state_update_ssu_amd.workloads import Workload


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def i64(t):
    return None if t is None else t.detach().to("cpu", torch.int64).numpy()


def bits(t):
    """Integer view of a tensor's bit pattern (exact comparisons, NaN-safe)."""
    view = {torch.float32: torch.int32, torch.float16: torch.int16,
            torch.bfloat16: torch.int16}[t.dtype]
    return t.view(view)


# ------------------------------------------------------------------ GPU side

def gpu_run(w: Workload, heads_per_block=0, loads_per_lane=0, tile_order=0):
    """Run the workload on its device. Returns (out, state_after, state_before);
    the workload's own state tensor is left untouched."""
    state = w.state.clone()
    out = w.out_sentinel()
    common = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                  pad_slot_id=w.pad_slot_id, disable_state_update=w.disable_state_update,
                  rand_seed=w.rand_seed, philox_rounds=w.philox_rounds,
                  heads_per_block=heads_per_block, loads_per_lane=loads_per_lane,
                  tile_order=tile_order)
    if w.mode == "one_token":
        ssu.ssu_one_token(state, w.x, w.dt, w.A, w.B, w.C, out,
                          state_batch_indices=w.src, dst_state_batch_indices=w.dst, **common)
    elif w.meta.get("dense"):
        # The dense [batch, steps, ...] layout: every operand 4-D, no starts tensor.
        nseq = w.cu_seqlens.shape[0] - 1
        d4 = lambda t: None if t is None else t.view(nseq, -1, *t.shape[1:])
        ret = ssu.ssu_packed_varlen(state, d4(w.x), d4(w.dt), w.A, d4(w.B), d4(w.C), None,
                                    d4(out), num_accepted_tokens=w.num_accepted,
                                    state_batch_indices=w.src_table,
                                    dst_state_batch_indices=w.dst_table,
                                    **dict(common, z=d4(w.z)))
        assert ret.data_ptr() == out.data_ptr() and ret.dim() == 4
    else:
        ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, w.cu_seqlens, out,
                              num_accepted_tokens=w.num_accepted,
                              state_batch_indices=w.src_table,
                              dst_state_batch_indices=w.dst_table,
                              steps=w.meta.get("steps"), **common)
    torch.cuda.synchronize()
    return out, state, w.state


# --------------------------------------------------------------- oracle side

def sr_args(w: Workload, rounding=True):
    """The oracle's stochastic-rounding arguments for a workload (none unless a
    seed is set and the state is 16-bit)."""
    if not rounding or w.rand_seed is None or w.state.dtype == torch.float32:
        return {}
    fmt = "bf16" if w.state.dtype == torch.bfloat16 else "f16"
    return dict(sr_format=fmt, rand_seed=int(w.rand_seed.item()), philox_rounds=w.philox_rounds)


def oracle_full(w: Workload, state=None, rounding=True):
    """The oracle on the whole workload (small problems). With rounding=False a
    stochastic-rounding workload is run without it (the unrounded states)."""
    orc = oracle.default()
    st = f64(w.state if state is None else state)
    common = dict(D=f64(w.D), z=f64(w.z), dt_bias=f64(w.dt_bias), dt_softplus=w.dt_softplus,
                  pad_slot_id=w.pad_slot_id, disable_state_update=w.disable_state_update,
                  **sr_args(w, rounding))
    if w.mode == "one_token":
        return orc.one_token(st, f64(w.x), f64(w.dt), f64(w.A), f64(w.B), f64(w.C),
                             src=i64(w.src), dst=i64(w.dst), **common)
    strides = w.meta.get("table_strides")
    return orc.packed_varlen(st, f64(w.x), f64(w.dt), f64(w.A), f64(w.B), f64(w.C),
                             i64(w.cu_seqlens), num_accepted=i64(w.num_accepted),
                             src_table=i64(w.src_table), src_strides=strides,
                             dst_table=i64(w.dst_table), dst_strides=strides,
                             steps=w.meta.get("steps"), **common)


def _valid(s, pad, nslots):
    return s != pad and 0 <= s < nslots


def oracle_sample(w: Workload, seqs, state_before, rounding=True):
    """The oracle on sequences `seqs` of a workload with 2-D (or no) tables.
    Returns (rows, out_ref [len(rows), H, P], slots, state_ref [len(slots), ...]):
    `rows` index the full out tensor, `slots` the full state cache. Stochastic
    rounding numbers its random bits by the call-wide packed row, so with a seed
    `seqs` must be a run of consecutive sequences, and the oracle is told the
    packed row where the run begins (sr_row_base)."""
    orc = oracle.default()
    sr = sr_args(w, rounding)
    if sr:
        seqs = list(seqs)
        assert seqs == list(range(seqs[0], seqs[0] + len(seqs))), \
            "stochastic rounding needs consecutive sequences"
        sr = dict(sr, sr_row_base=(seqs[0] if w.mode == "one_token"
                                   else int(i64(w.cu_seqlens)[seqs[0]])))
    nslots = w.state.shape[0]
    pad = w.pad_slot_id
    seqs = list(seqs)
    if w.mode == "one_token":
        src = i64(w.src)
        dst = i64(w.dst)
        r = [int(src[b]) if src is not None else b for b in seqs]
        d = [int(dst[b]) if dst is not None else r[i] for i, b in enumerate(seqs)]
        used = sorted({s for s in r + d if _valid(s, pad, nslots)})
        remap = {s: i for i, s in enumerate(used)}
        rs = np.array([remap.get(s, -1) for s in r])
        ds = np.array([remap.get(s, -1) for s in d])
        rows = np.array(seqs)
        sub_state = f64(state_before[torch.as_tensor(used, dtype=torch.long,
                                                    device=state_before.device)])
        if not used:
            sub_state = np.zeros((1,) + tuple(w.state.shape[1:]))
        res = orc.one_token(sub_state, f64(w.x[rows]), f64(w.dt[rows]), f64(w.A),
                            f64(w.B[rows]), f64(w.C[rows]), D=f64(w.D),
                            z=None if w.z is None else f64(w.z[rows]), dt_bias=f64(w.dt_bias),
                            dt_softplus=w.dt_softplus, src=rs, dst=ds, pad_slot_id=-1,
                            disable_state_update=w.disable_state_update, **sr)
        return rows, res.out, used, res.state[:len(used)]

    cu = i64(w.cu_seqlens)
    total = w.rows
    rows, sub_cu = [], [0]
    for b in seqs:
        lo, hi = int(cu[b]), int(cu[b + 1])
        if lo < 0 or hi > total or hi < lo:
            lo = hi = 0
        rows.extend(range(lo, hi))
        sub_cu.append(len(rows))
    rows = np.array(rows, dtype=np.int64)
    st = i64(w.src_table)
    dt_ = i64(w.dst_table)
    tabs = [t[seqs] for t in (st, dt_) if t is not None]
    used = sorted({int(s) for t in tabs for s in t.reshape(-1) if _valid(int(s), pad, nslots)})
    if st is None:
        used = sorted(set(used) | {b for b in seqs if _valid(b, pad, nslots)})
    remap = {s: i for i, s in enumerate(used)}

    def rm(t):
        if t is None:
            return None
        return np.vectorize(lambda s: remap.get(int(s), -1), otypes=[np.int64])(t[seqs])

    sub_src = rm(st)
    if st is None and seqs != list(range(len(seqs))):
        # Identity read slots: sequence b reads slot b; express that as a table.
        sub_src = np.array([[remap.get(b, -1)] for b in seqs], dtype=np.int64)
    sub_dst = rm(dt_)
    na = i64(w.num_accepted)
    sub_na = None if na is None else na[seqs]
    if sub_src is not None and st is None and sub_na is not None:
        raise ValueError("acceptance counts need a read table")
    steps = w.meta.get("steps")
    if steps is None:
        steps = (st if st is not None else dt_).shape[1] if (st is not None or dt_ is not None) else 1
    sub_state = (f64(state_before[torch.as_tensor(used, dtype=torch.long,
                                                  device=state_before.device)])
                 if used else np.zeros((1,) + tuple(w.state.shape[1:])))
    sel = torch.as_tensor(rows, dtype=torch.long, device=w.x.device)
    res = orc.packed_varlen(
        sub_state, f64(w.x[sel]), f64(w.dt[sel]), f64(w.A), f64(w.B[sel]), f64(w.C[sel]),
        np.array(sub_cu), num_accepted=sub_na,
        src_table=sub_src, dst_table=sub_dst, steps=steps if (sub_src is not None or sub_dst is not None) else None,
        D=f64(w.D), z=None if w.z is None else f64(w.z[sel]), dt_bias=f64(w.dt_bias),
        dt_softplus=w.dt_softplus, pad_slot_id=-1, disable_state_update=w.disable_state_update,
        **sr)
    return rows, res.out, used, res.state[:len(used)]


# ---------------------------------------------------------------- comparison

def tolerance_check(name, got: torch.Tensor, ref: np.ndarray):
    """Compare a GPU tensor with an fp64 reference at the dtype's tolerance.
    NaN in the reference marks elements the call must leave alone; those are
    checked by the caller against the sentinel, and skipped here."""
    g = f64(got)
    mask = ~np.isnan(ref)
    if not mask.any():
        return 0.0
    g, r = g[mask], ref[mask]
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values where the reference is finite"
    err = np.abs(g - r)
    if got.dtype == torch.float32:
        scale = max(1.0, float(np.max(np.abs(r))))
        worst = float(err.max())
        assert worst <= 1e-5 * scale, f"{name}: fp32 max abs err {worst:.3e} > 1e-5 * {scale:.3e}"
        return worst / scale
    bound = 1e-2 + 2e-2 * np.abs(r)
    ratio = float((err / bound).max())
    assert ratio <= 1.0, (f"{name}: {got.dtype} error exceeds 1e-2 + 2e-2|ref| "
                          f"(worst ratio {ratio:.3f}, max err {float(err.max()):.3e})")
    return ratio


def check_out_rows(name, out_gpu: torch.Tensor, rows, out_ref: np.ndarray):
    """Rows the reference wrote must match at tolerance; rows it left alone
    (NaN) must still hold the NaN sentinel bit for bit on the GPU."""
    got = out_gpu[torch.as_tensor(rows, dtype=torch.long, device=out_gpu.device)]
    untouched = np.isnan(out_ref)
    if untouched.any():
        sentinel = bits(torch.full((), float("nan"), dtype=out_gpu.dtype)).item()
        g_bits = bits(got.cpu()).numpy()
        assert np.all(g_bits[untouched] == sentinel), f"{name}: GPU wrote rows the reference did not"
    return tolerance_check(name, got, out_ref)


def check_slots(name, state_after: torch.Tensor, state_before: torch.Tensor, slots,
                state_ref: np.ndarray):
    """Slots the reference leaves unchanged must be bit-identical on the GPU;
    the others must match at tolerance."""
    if not len(slots):
        return 0.0
    idx = torch.as_tensor(slots, dtype=torch.long, device=state_after.device)
    after = state_after[idx]
    before = state_before[idx]
    ref_unchanged = np.array([np.array_equal(state_ref[i], f64(before[i])) for i in range(len(slots))])
    worst = 0.0
    for i, s in enumerate(slots):
        if ref_unchanged[i]:
            assert torch.equal(bits(after[i]), bits(before[i])), f"{name}: slot {s} changed on the GPU"
        else:
            worst = max(worst, tolerance_check(f"{name} slot {s}", after[i], state_ref[i]))
    return worst


def changed_slots(state_after: torch.Tensor, state_before: torch.Tensor):
    """Slots whose bytes differ (computed on the device)."""
    a = bits(state_after).reshape(state_after.shape[0], -1)
    b = bits(state_before).reshape(state_before.shape[0], -1)
    return torch.nonzero((a != b).any(dim=1)).flatten().cpu().tolist()


def oracle_placement(w: Workload):
    """Which slots the call writes and which out rows it leaves alone, from the
    oracle run on a shadow problem: the workload's own slot vectors / tables,
    cu_seqlens and acceptance counts, with one head, one row and one state
    element. Slot s starts at s + 0.5 and every step maps a value v to
    v / e + 1, so no written value equals any slot's starting value and the
    slots that change are exactly the slots written.
    Returns (written slot set, boolean [rows] mask of untouched out rows)."""
    orc = oracle.default()
    nslots, rows = w.state.shape[0], w.rows
    state = (np.arange(nslots, dtype=np.float64) + 0.5).reshape(nslots, 1, 1, 1)
    ones = np.ones((rows, 1, 1))
    common = dict(dt_softplus=False, pad_slot_id=w.pad_slot_id,
                  disable_state_update=w.disable_state_update)
    args = (state, ones, np.ones((rows, 1)), np.array([-1.0]), ones, ones)
    if w.mode == "one_token":
        res = orc.one_token(*args, src=i64(w.src), dst=i64(w.dst), **common)
    else:
        strides = w.meta.get("table_strides")
        res = orc.packed_varlen(*args, i64(w.cu_seqlens), num_accepted=i64(w.num_accepted),
                                src_table=i64(w.src_table), src_strides=strides,
                                dst_table=i64(w.dst_table), dst_strides=strides,
                                steps=w.meta.get("steps"), **common)
    written = {int(s) for s in np.nonzero(res.state[:, 0, 0, 0] != state[:, 0, 0, 0])[0]}
    return written, np.isnan(res.out[:, 0, 0])


def check_placement(name, w: Workload, out_gpu, state_after, state_before):
    """Exact placement over the whole call: the changed slots are exactly the
    written ones, untouched out rows keep the sentinel, the others are finite."""
    written, untouched = oracle_placement(w)
    changed = set(changed_slots(state_after, state_before))
    assert changed == written, (f"{name}: slots changed on the GPU differ from the slots "
                                f"written: extra {sorted(changed - written)[:8]}, "
                                f"missing {sorted(written - changed)[:8]}")
    sentinel = bits(torch.full((), float("nan"), dtype=out_gpu.dtype)).item()
    ob = bits(out_gpu).reshape(out_gpu.shape[0], -1)
    kept = (ob == sentinel).all(dim=1).cpu().numpy()
    assert np.array_equal(kept, untouched), (
        f"{name}: out rows left alone on the GPU differ from the reference "
        f"({int(kept.sum())} vs {int(untouched.sum())})")
    live = torch.as_tensor(~untouched, device=out_gpu.device)
    assert torch.isfinite(out_gpu[live].float()).all(), f"{name}: non-finite values in written out rows"
    return written, untouched


def _neighbours(v, dtype):
    """The two values of a 16-bit format bracketing each v (toward and away from
    zero), from torch's rounding and the adjacent bit patterns."""
    n = torch.tensor(v).to(torch.float32).to(dtype)
    nb = n.view(torch.int16).numpy().astype(np.int32)
    nv = n.double().numpy()
    up = torch.tensor((nb + 1).astype(np.int16)).view(dtype).double().numpy()
    dn = torch.tensor(np.maximum(nb - 1, nb & ~0x7FFF).astype(np.int16)).view(dtype).double().numpy()
    toward = np.where(np.abs(nv) <= np.abs(v), nv, dn)
    away = np.where(np.abs(nv) <= np.abs(v), np.where(nv == v, nv, up), nv)
    return toward, away


def check_slots_sr(name, state_after, state_before, slots, state_sr, state_plain,
                   max_flip_rate=2e-3):
    """Stochastically rounded slots: the GPU value equals the oracle's
    stochastic rounding (same random words) except where the GPU's fp32 state and
    the oracle's fp64 state fall on opposite sides of a rounding threshold. Such
    elements must be rare and, like every element, within the 16-bit tolerance of
    the exact state (near-zero states from cancellation can sit several 16-bit
    spacings from their fp32 value). Slots the oracle leaves unchanged must be
    bit-identical."""
    idx = torch.as_tensor(slots, dtype=torch.long, device=state_after.device)
    after = f64(state_after[idx])
    before = f64(state_before[idx])
    flips = total = 0
    for i, s in enumerate(slots):
        if np.array_equal(state_sr[i], before[i]) and np.array_equal(state_plain[i], before[i]):
            assert np.array_equal(after[i], before[i]), f"{name}: slot {s} changed on the GPU"
            continue
        g, want, exact = after[i].reshape(-1), state_sr[i].reshape(-1), state_plain[i].reshape(-1)
        bad = g != want
        err = np.abs(g - exact)
        ratio = float((err / (1e-2 + 2e-2 * np.abs(exact))).max())
        assert ratio <= 1.0, f"{name}: slot {s}: error beyond the 16-bit tolerance ({ratio:.3f})"
        flips += int(bad.sum())
        total += g.size
    rate = flips / max(total, 1)
    assert rate <= max_flip_rate, f"{name}: {flips} of {total} elements rounded the other way"
    return rate
