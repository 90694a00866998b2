"""GPU path against the fp64 oracle, through the C ABI (via the binding).

Small shapes (spanning several workgroups and a ragged row block) are compared
in full; the named decode workloads run at their real sizes, in the launch
configuration the benchmark times, with exact placement checked over the whole
call and every sequence compared against the oracle."""
import itertools
import sys

import numpy as np
import pytest
import torch

import harness as hz
from selective_state_update_ssu_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare_full(name, w, out, after, before, ref):
    hz.check_placement(name, w, out, after, before)
    e_out = hz.check_out_rows(name + " out", out, np.arange(w.rows), ref.out)
    e_st = hz.check_slots(name + " state", after, before, list(range(w.state.shape[0])), ref.state)
    return e_out, e_st


# ----------------------------------------------------------- named workloads

def _runs(n, size):
    return [list(range(b, min(b + size, n))) for b in range(0, n, size)]


@pytest.mark.parametrize("name", list(wl.NAMED))
def test_named_workload(name):
    """The full-size workload in the benchmark's launch configuration: exact
    placement over the whole call, and every sequence compared against the
    oracle (runs of 32 consecutive sequences, each cut out with its slots)."""
    _say(f"[parity] named workload {name}")
    w = wl.NAMED[name](DEV)
    out, after, before = hz.gpu_run(w)
    written, untouched = hz.check_placement(name, w, out, after, before)
    n = w.rows if w.mode == "one_token" else w.cu_seqlens.shape[0] - 1
    worst_out = worst_st = 0.0
    compared = 0
    for seqs in _runs(n, 32):
        rows, out_ref, slots, state_ref = hz.oracle_sample(w, seqs, before)
        e_out = hz.check_out_rows(f"{name} out (sequences {seqs[0]}..{seqs[-1]})", out, rows,
                                  out_ref)
        if hz.sr_args(w):
            _, _, _, state_plain = hz.oracle_sample(w, seqs, before, rounding=False)
            e_st = hz.check_slots_sr(f"{name} state", after, before, slots, state_ref,
                                     state_plain)
        else:
            e_st = hz.check_slots(f"{name} state", after, before, slots, state_ref)
        worst_out, worst_st = max(worst_out, e_out), max(worst_st, e_st)
        compared += len(seqs)
    assert compared == n
    _say(f"[parity] {name}: {compared} of {n} sequences compared ({n - int(untouched.sum())} "
         f"rows written, {len(written)} slots written, {int(untouched.sum())} rows inert); "
         f"worst out {worst_out:.3g}, worst state {worst_st:.3g}"
         + (" (stochastic rounding: share of threshold flips)" if hz.sr_args(w) else ""))


@pytest.mark.parametrize("name", ["nemotron_h", "packed_mtp", "bf16_state"])
def test_launch_shapes_bit_identical(name):
    """The launch shape (heads per workgroup, loads per lane, tile order) changes
    nothing in the arithmetic of an element: every shape gives the same bits."""
    w = wl.NAMED[name](DEV)
    o1, s1, _ = hz.gpu_run(w, heads_per_block=1, loads_per_lane=2, tile_order=2)
    shapes = ((2, 2), (4, 1), (4, 2)) if w.mode == "packed" else ((2, 2), (2, 4), (4, 1), (4, 2), (4, 4))
    for order in (1, 2, 3):
        for lpl, hpb in shapes:
            o2, s2, _ = hz.gpu_run(w, heads_per_block=hpb, loads_per_lane=lpl, tile_order=order)
            assert torch.equal(hz.bits(o1), hz.bits(o2)), (lpl, hpb, order)
            assert torch.equal(hz.bits(s1), hz.bits(s2)), (lpl, hpb, order)
            del o2, s2



@pytest.mark.parametrize("state_dtype,N", [("bf16", 16), ("f16", 16), ("f32", 16), ("bf16", 32)])
@pytest.mark.parametrize("mode", ["one_token", "packed"])
def test_short_row_launch_shapes(state_dtype, N, mode):
    """dstate rows of 64 bytes or less take one- or two-wave head groups whose
    lanes hold two to four rows: every (loads_per_lane, heads_per_block, tile
    order) gives the same bits, and those bits match the oracle. headdim 72
    leaves a ragged second row block."""
    if mode == "one_token":
        w = wl.one_token("short", 111, batch=9, H=8, P=72, N=N, G=2, nslots=24, device=DEV,
                         state_dtype=state_dtype, io="bf16", pad_fraction=0.2,
                         dst_mode="distinct")
    else:
        w = wl.packed("short", 112, nseq=7, max_len=12, H=8, P=72, N=N, G=2, nslots=90,
                      device=DEV, state_dtype=state_dtype, lengths=[3, 1, 12, 0, 9, 4, 1],
                      pad_fraction=0.15)
    o1, s1, before = hz.gpu_run(w, heads_per_block=1, loads_per_lane=2, tile_order=2)
    compare_full(f"short-{mode}-{state_dtype}-{N}", w, o1, s1, before, hz.oracle_full(w))
    hpbs = (1, 2) if mode == "packed" else (1, 2, 4)
    for lpl, hpb, order in itertools.product((2, 4), hpbs, (1, 2, 3)):
        o2, s2, _ = hz.gpu_run(w, heads_per_block=hpb, loads_per_lane=lpl, tile_order=order)
        assert torch.equal(hz.bits(o1), hz.bits(o2)), (lpl, hpb, order)
        assert torch.equal(hz.bits(s1), hz.bits(s2)), (lpl, hpb, order)


# ---------------------------------------------------------------- small grid

def _small_cases():
    cases = []
    for st, io in itertools.product(["f32", "f16", "bf16"], ["f32", "f16", "bf16"]):
        cases.append(dict(state_dtype=st, io=io, N=128, P=64, H=8, G=2))
    for N in (16, 32, 64, 256):
        for st in ("f32", "bf16"):
            cases.append(dict(state_dtype=st, io="bf16", N=N, P=64, H=4, G=1))
    for P in (80, 40, 128, 1):
        cases.append(dict(state_dtype="f32", io="bf16", N=64, P=P, H=4, G=2))
    # headdim 256 (several row blocks per head at every geometry); one head
    cases.append(dict(state_dtype="bf16", io="bf16", N=128, P=256, H=2, G=1))
    cases.append(dict(state_dtype="f16", io="f16", N=16, P=256, H=2, G=2))
    cases.append(dict(state_dtype="f32", io="bf16", N=128, P=64, H=1, G=1))
    cases.append(dict(state_dtype="f16", io="f16", N=16, P=72, H=6, G=3))
    # launch shapes, optional operands and index dtypes
    cases.append(dict(state_dtype="f32", io="bf16", N=128, P=64, H=8, G=1, hpb=4))
    cases.append(dict(state_dtype="bf16", io="f16", N=128, P=64, H=8, G=2, hpb=2))
    cases.append(dict(state_dtype="f32", io="f16", N=256, P=64, H=4, G=1, hpb=2))
    cases.append(dict(state_dtype="f32", io="bf16", N=64, P=64, H=4, G=1, with_z=False,
                      with_D=False, with_bias=False))
    cases.append(dict(state_dtype="f32", io="bf16", N=64, P=64, H=4, G=1, dt_per_dim=True))
    cases.append(dict(state_dtype="f32", io="bf16", N=64, P=64, H=4, G=1, softplus=False))
    cases.append(dict(state_dtype="f16", io="bf16", N=32, P=64, H=4, G=4, index_dtype="i64",
                      pad_fraction=0.3, dst_mode="distinct"))
    cases.append(dict(state_dtype="f32", io="f32", N=16, P=64, H=8, G=1, dst_mode="none"))
    cases.append(dict(state_dtype="f32", io="bf16", N=128, P=64, H=4, G=1, identity=True))
    cases.append(dict(state_dtype="f32", io="bf16", N=128, P=64, H=4, G=1, disable=True,
                      pad_fraction=0.2))
    return cases


def _case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


def _one_token_case(c, seed):
    c = dict(c)
    batch = c.pop("batch", 7)
    hpb = c.pop("hpb", 0)
    disable = c.pop("disable", False)
    softplus = c.pop("softplus", True)
    nslots = c.pop("nslots", 2 * batch + 3)
    w = wl.one_token("small", seed, batch=batch, nslots=nslots, device=DEV, **c)
    w.dt_softplus = softplus
    w.disable_state_update = disable
    return w, hpb


@pytest.mark.parametrize("case", _small_cases(), ids=_case_id)
def test_one_token_small(case):
    w, hpb = _one_token_case(case, seed=101)
    out, after, before = hz.gpu_run(w, heads_per_block=hpb)
    ref = hz.oracle_full(w)
    compare_full(_case_id(case), w, out, after, before, ref)


@pytest.mark.parametrize("case", [
    dict(state_dtype="f32", io="bf16", N=128, P=64, H=8, G=2),
    dict(state_dtype="bf16", io="f16", N=64, P=80, H=4, G=1),
    dict(state_dtype="f16", io="f32", N=16, P=64, H=4, G=2, hpb=2),
    dict(state_dtype="f32", io="bf16", N=256, P=64, H=4, G=1, meta_dtype="i64", index_dtype="i64"),
    dict(state_dtype="f32", io="bf16", N=128, P=64, H=4, G=1, accepted=False),
    dict(state_dtype="f32", io="bf16", N=64, P=64, H=4, G=1, with_z=False, dt_per_dim=True),
    dict(state_dtype="f32", io="bf16", N=128, P=64, H=4, G=1, disable=True),
    dict(state_dtype="bf16", io="bf16", N=64, P=256, H=2, G=1),
    dict(state_dtype="f32", io="f32", N=32, P=64, H=1, G=1),
], ids=_case_id)
def test_packed_small(case):
    c = dict(case)
    hpb = c.pop("hpb", 0)
    disable = c.pop("disable", False)
    lengths = [1, 4, 0, 2, 3, 1, 0, 4, 2]          # includes empty sequences
    w = wl.packed("small", 202, nseq=len(lengths), max_len=4, nslots=48, device=DEV,
                  lengths=lengths, pad_fraction=0.12, **c)
    w.disable_state_update = disable
    out, after, before = hz.gpu_run(w, heads_per_block=hpb)
    ref = hz.oracle_full(w)
    compare_full(_case_id(case), w, out, after, before, ref)


@pytest.mark.parametrize("case", [
    dict(state_dtype="f32", io="bf16", N=128, P=64, H=4, G=1),
    dict(state_dtype="bf16", io="f16", N=64, P=80, H=4, G=2, hpb=2),
    dict(state_dtype="f16", io="f32", N=256, P=64, H=2, G=1),
    dict(state_dtype="f32", io="bf16", N=16, P=64, H=4, G=4, accepted=False),
], ids=_case_id)
def test_packed_sequences_longer_than_a_staged_chunk(case):
    """Sequences of 8, 9, 16, 17 and 23 tokens: the kernel stages the per-token
    operands eight tokens at a time, so these cross one, two and three restaging
    points with the state still in registers; every token's destination is
    checked."""
    c = dict(case)
    hpb = c.pop("hpb", 0)
    lengths = [9, 1, 17, 8, 0, 23, 16, 2]
    w = wl.packed("long", 212, nseq=len(lengths), max_len=24, nslots=200, device=DEV,
                  lengths=lengths, pad_fraction=0.12, **c)
    out, after, before = hz.gpu_run(w, heads_per_block=hpb)
    compare_full(_case_id(case), w, out, after, before, hz.oracle_full(w))


def test_dense_sequences_longer_than_a_staged_chunk():
    """A dense [batch, 11, heads, dim] call: every sequence restages its operands
    once, at token 8."""
    w = wl.packed("denselong", 213, nseq=5, max_len=11, H=4, P=64, N=128, G=1, nslots=64,
                  device=DEV, dense=True, pad_fraction=0.2)
    out, after, before = hz.gpu_run(w)
    compare_full("dense-long", w, out, after, before, hz.oracle_full(w))


def test_pad_slot_id_inside_the_cache_and_wide_slot_ids():
    """pad_slot_id may name a real slot: a sequence reading it is inert and a
    write to it is dropped, while -1 and int64 ids beyond the cache (2^40,
    -2^40) are out of range and act as pads too."""
    w = wl.one_token("padid", 121, batch=12, H=4, P=64, N=64, G=1, nslots=30, device=DEV,
                     index_dtype="i64", dst_mode="distinct")
    pad = int(w.src[3])
    w.pad_slot_id = pad
    w.dst[5] = pad
    w.src[7] = -1
    w.src[8] = 1 << 40
    w.dst[9] = -(1 << 40)
    out, after, before = hz.gpu_run(w)
    compare_full("pad-id one-token", w, out, after, before, hz.oracle_full(w))
    assert torch.equal(hz.bits(after[pad]), hz.bits(before[pad]))

    p = wl.packed("padid", 122, nseq=6, max_len=4, H=4, P=64, N=64, G=1, nslots=40,
                  device=DEV, index_dtype="i64", lengths=[3, 4, 1, 2, 4, 2])
    pad = int(p.src_table[1, 0])
    p.pad_slot_id = pad
    p.src_table[4, 2] = 1 << 40
    p.src_table[5, 1] = -1
    out, after, before = hz.gpu_run(p)
    compare_full("pad-id packed", p, out, after, before, hz.oracle_full(p))
    assert torch.equal(hz.bits(after[pad]), hz.bits(before[pad]))


# ------------------------------------------------------------- packed edges

def _packed_base(seed=303, **kw):
    lengths = [3, 1, 2, 4]
    return wl.packed("edge", seed, nseq=4, max_len=4, H=4, P=64, N=64, G=1, nslots=24,
                     device=DEV, lengths=lengths, **kw)


def test_packed_write_back_without_destination_table():
    w = _packed_base()
    w.dst_table = None
    out, after, before = hz.gpu_run(w)
    compare_full("no-dst", w, out, after, before, hz.oracle_full(w))


def test_packed_identity_read_without_tables():
    w = _packed_base(accepted=False)
    w.src_table = None
    w.dst_table = None
    out, after, before = hz.gpu_run(w)
    compare_full("no-tables", w, out, after, before, hz.oracle_full(w))


def test_packed_steps_narrower_than_sequences():
    """Positions at or beyond the table width are not written; counts beyond it
    make the sequence inert."""
    w = _packed_base()
    w.src_table = w.src_table[:, :2].contiguous()
    w.dst_table = w.src_table
    w.num_accepted = torch.tensor([1, 1, 2, 3], dtype=w.cu_seqlens.dtype, device=DEV)
    out, after, before = hz.gpu_run(w)
    compare_full("narrow", w, out, after, before, hz.oracle_full(w))


def test_packed_flat_tables():
    """A flat per-row table addresses entry b + t (strides 1, 1)."""
    lengths = [1, 1, 1, 1, 1]
    w = wl.packed("flat", 404, nseq=5, max_len=1, H=4, P=64, N=32, G=1, nslots=16,
                  device=DEV, lengths=lengths, accepted=False)
    flat = torch.tensor([7, 3, 12, -1, 5], dtype=torch.int32, device=DEV)
    w.src_table = flat
    w.dst_table = flat
    w.meta["steps"] = 1
    w.meta["table_strides"] = (1, 1)
    out, after, before = hz.gpu_run(w)
    compare_full("flat", w, out, after, before, hz.oracle_full(w))


def test_packed_bad_row_ranges_are_inert():
    w = _packed_base()
    cu = w.cu_seqlens.clone()
    cu[2] = cu[3] + 1           # sequence 1 runs backwards, sequence 2 starts late
    cu[4] = w.rows + 5          # sequence 3 runs past the rows
    w.cu_seqlens = cu
    out, after, before = hz.gpu_run(w)
    compare_full("bad-ranges", w, out, after, before, hz.oracle_full(w))


def test_packed_bad_counts_and_slots_are_inert():
    w = _packed_base()
    w.num_accepted = torch.tensor([0, 5, -3, 2], dtype=w.cu_seqlens.dtype, device=DEV)
    t = w.src_table.clone()
    t[3, 1] = 10_000            # out-of-range read slot for sequence 3
    t[0, 2] = -1                # pad destination at position 2 of sequence 0
    w.src_table = t
    w.dst_table = t
    out, after, before = hz.gpu_run(w)
    compare_full("bad-counts", w, out, after, before, hz.oracle_full(w))


# ------------------------------------------------------------ exact copies

@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_zero_step_copies_slot_bit_exact(state_dtype):
    """dt + dt_bias = 0 with softplus off: the destination slot is a bit-exact
    copy of the source slot, in every storage dtype."""
    w = wl.one_token("copy", 505, batch=6, H=4, P=64, N=128, G=1, nslots=16, device=DEV,
                     state_dtype=state_dtype, io="bf16", dst_mode="distinct")
    w.dt_softplus = False
    w.dt = -w.dt_bias.expand(w.rows, -1).contiguous()
    out, after, before = hz.gpu_run(w)
    for b in range(w.rows):
        s, d = int(w.src[b]), int(w.dst[b])
        assert torch.equal(hz.bits(after[d]), hz.bits(before[s])), b
    compare_full("copy", w, out, after, before, hz.oracle_full(w))


# ------------------------------------------------------------- empty calls

def test_empty_calls_launch_nothing():
    import selective_state_update_ssu_amd as ssu
    w = wl.one_token("empty", 606, batch=0, H=4, P=64, N=64, G=1, nslots=4, device=DEV)
    out = ssu.ssu_one_token(w.state, w.x, w.dt, w.A, w.B, w.C, D=w.D, z=w.z,
                            dt_bias=w.dt_bias, state_batch_indices=w.src)
    assert out.shape[0] == 0
    p = _packed_base()
    cu = torch.zeros(3, dtype=torch.int32, device=DEV)
    x = p.x[:0]
    ssu.ssu_packed_varlen(p.state, x, p.dt[:0], p.A, p.B[:0], p.C[:0], cu, D=p.D,
                          z=p.z[:0], dt_bias=p.dt_bias)
    torch.cuda.synchronize()


# ------------------------------------------------------------ dense layout

@pytest.mark.parametrize("case", [
    dict(state_dtype="f32", io="bf16", N=128, P=64, H=8, G=2),
    dict(state_dtype="bf16", io="f16", N=64, P=80, H=4, G=1, accepted=False),
], ids=_case_id)
def test_dense_layout(case):
    """[batch, steps, heads, dim] operands run as regular sequences (no starts
    tensor): equal to the oracle given the regular starts, and bit-identical to
    the packed call with an explicit cu_seqlens."""
    w = wl.packed("dense", 707, nseq=6, max_len=3, nslots=24, device=DEV, dense=True,
                  pad_fraction=0.2, **case)
    out, after, before = hz.gpu_run(w)
    compare_full("dense", w, out, after, before, hz.oracle_full(w))
    w.meta["dense"] = False
    out2, after2, _ = hz.gpu_run(w)
    assert torch.equal(hz.bits(out), hz.bits(out2))
    assert torch.equal(hz.bits(after), hz.bits(after2))


def test_packed_one_row_per_sequence_without_starts():
    """Without cu_seqlens a packed x holds one row per sequence."""
    import selective_state_update_ssu_amd as ssu
    w = wl.packed("onerow", 808, nseq=7, max_len=2, H=4, P=64, N=64, G=1, nslots=16,
                  device=DEV, lengths=[1] * 7, pad_fraction=0.15)
    ref = hz.oracle_full(w)
    state = w.state.clone()
    out = w.out_sentinel()
    ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, None, out, D=w.D, z=w.z,
                          dt_bias=w.dt_bias, dt_softplus=True,
                          num_accepted_tokens=w.num_accepted, state_batch_indices=w.src_table,
                          dst_state_batch_indices=w.dst_table)
    torch.cuda.synchronize()
    compare_full("onerow", w, out, state, w.state, ref)


@pytest.mark.parametrize("form", ["hpn_all_zero", "hp_zero", "hpn_last_zero_p1", "column"])
def test_tied_parameter_views_bit_identical(form):
    """Per-head A/D/dt_bias given as tied views give the same bits as [heads]
    vectors: [heads, dim, dstate] with both inner strides 0, [heads, dim] with
    stride 0 along dim, [heads, 1, dstate] with stride 0 along dstate, and
    [heads, 1] columns; dt as a [rows, heads, dim] view with stride 0 along dim
    gives the bits of the [rows, heads] dt."""
    w = wl.one_token("tied", 909, batch=5, H=4, P=64, N=128, G=1, nslots=12, device=DEV)
    o1, s1, _ = hz.gpu_run(w)
    H, P, N = 4, 64, 128
    if form == "hpn_all_zero":
        w.A = w.A[:, None, None].expand(H, P, N)
        w.dt_bias = w.dt_bias[:, None, None].expand(H, P, N)
        w.D = w.D[:, None].contiguous()
    elif form == "hp_zero":
        w.A = w.A[:, None].expand(H, P)
        w.D = w.D[:, None].expand(H, P)
        w.dt_bias = w.dt_bias[:, None].expand(H, P)
        w.dt = w.dt[:, :, None].expand(w.rows, H, P)
    elif form == "hpn_last_zero_p1":
        w.D = w.D[:, None, None].expand(H, 1, N)
        w.dt_bias = w.dt_bias[:, None, None].expand(H, 1, N)
    else:
        w.A, w.D, w.dt_bias = (t[:, None].contiguous() for t in (w.A, w.D, w.dt_bias))
    o2, s2, _ = hz.gpu_run(w)
    assert torch.equal(hz.bits(o1), hz.bits(o2)) and torch.equal(hz.bits(s1), hz.bits(s2))


# ------------------------------------------------------- stochastic rounding

@pytest.mark.parametrize("state_dtype,mode,rounds", [("bf16", "one_token", 10),
                                                      ("f16", "one_token", 10),
                                                      ("bf16", "packed", 7),
                                                      ("f16", "packed", 10),
                                                      ("bf16", "packed_long", 10),
                                                      ("bf16", "one_token_d16", 10),
                                                      ("f16", "one_token_d16", 10),
                                                      ("bf16", "packed_d32", 10),
                                                      ("f16", "packed_d32", 10)])
def test_stochastic_rounding(state_dtype, mode, rounds):
    """Stored 16-bit states equal the oracle's stochastic rounding with the same
    Philox words (up to rare threshold flips between the fp32 and fp64 states);
    out and placement are those of the round-to-nearest call. dstate 16 and 32
    run the short-row geometry (two or four rows per lane)."""
    if mode in ("one_token", "one_token_d16"):
        N = 16 if mode == "one_token_d16" else 128
        w = wl.one_token("sr", 1001, batch=9, H=8, P=64, N=N, G=2, nslots=24, device=DEV,
                         state_dtype=state_dtype, io="bf16", pad_fraction=0.2,
                         dst_mode="distinct")
    elif mode in ("packed", "packed_d32"):
        N = 32 if mode == "packed_d32" else 64
        w = wl.packed("sr", 1002, nseq=7, max_len=4, H=4, P=64, N=N, G=1, nslots=40,
                      device=DEV, state_dtype=state_dtype, lengths=[3, 1, 4, 0, 2, 4, 1],
                      pad_fraction=0.15)
    else:  # sequences past the eight-token operand stage; rows number the draws
        w = wl.packed("srlong", 1004, nseq=4, max_len=19, H=4, P=64, N=128, G=1, nslots=90,
                      device=DEV, state_dtype=state_dtype, lengths=[9, 2, 19, 16])
    w.rand_seed = torch.tensor([0x0123_4567_89AB_CDEF], dtype=torch.int64, device=DEV)
    w.philox_rounds = rounds
    out, after, before = hz.gpu_run(w)
    hz.check_placement("sr", w, out, after, before)
    ref_sr = hz.oracle_full(w)
    ref_plain = hz.oracle_full(w, rounding=False)
    hz.check_out_rows("sr out", out, np.arange(w.rows), ref_plain.out)
    rate = hz.check_slots_sr("sr state", after, before, list(range(w.state.shape[0])),
                             ref_sr.state, ref_plain.state)
    seed = w.rand_seed
    w.rand_seed = None
    out_rne, _, _ = hz.gpu_run(w)
    assert torch.equal(hz.bits(out), hz.bits(out_rne))
    _say(f"[parity] stochastic rounding {state_dtype} {mode}: flip rate {rate:.2e}")
    del seed


def test_stochastic_rounding_leaves_fp32_state_alone():
    w = wl.one_token("sr32", 1003, batch=5, H=4, P=64, N=128, G=1, nslots=12, device=DEV)
    o1, s1, _ = hz.gpu_run(w)
    w.rand_seed = torch.tensor([99], dtype=torch.int64, device=DEV)
    o2, s2, _ = hz.gpu_run(w)
    assert torch.equal(hz.bits(o1), hz.bits(o2)) and torch.equal(hz.bits(s1), hz.bits(s2))


def test_stochastic_rounding_is_unbiased_on_average():
    """Averaged over 64 seeds, the stored bf16 state of a fixed update is closer to
    the fp32 state than its round-to-nearest value is, on average."""
    w = wl.one_token("srmean", 1004, batch=4, H=4, P=64, N=128, G=1, nslots=8, device=DEV,
                     state_dtype="bf16", io="bf16", dst_mode="distinct")
    w32 = wl.one_token("srmean", 1004, batch=4, H=4, P=64, N=128, G=1, nslots=8, device=DEV,
                       state_dtype="bf16", io="bf16", dst_mode="distinct")
    w32.state = w32.state.float()
    _, exact, _ = hz.gpu_run(w32)
    _, rne, _ = hz.gpu_run(w)
    dst = w.dst.long()
    acc = torch.zeros_like(exact[dst])
    for k in range(64):
        w.rand_seed = torch.tensor([1000 + k], dtype=torch.int64, device=DEV)
        _, sr, _ = hz.gpu_run(w)
        acc += sr[dst].float()
    mean_err = (acc / 64 - exact[dst]).abs().mean().item()
    rne_err = (rne[dst].float() - exact[dst]).abs().mean().item()
    assert mean_err < 0.5 * rne_err, (mean_err, rne_err)


# ------------------------------------------------------------- concurrency

def test_threads_and_streams_match_a_single_thread():
    """Two host threads, each on its own HIP stream (default priority), each
    running a chain of in-place one-token and packed steps on a state cache of
    its own: every result equals the same chain run on one thread, bit for
    bit. The library keeps no state between calls (its error text is per
    thread), so concurrent callers cannot disturb each other."""
    import threading

    steps = 6
    works = [wl.one_token("conc1", 1101, batch=48, H=8, P=64, N=128, G=2, nslots=64,
                          device=DEV, pad_fraction=0.1),
             wl.packed("conc2", 1102, nseq=24, max_len=4, H=8, P=64, N=128, G=1,
                       nslots=128, device=DEV, pad_fraction=0.1)]

    import selective_state_update_ssu_amd as ssu

    def chain(w, state, out, stream=None):
        common = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                      pad_slot_id=w.pad_slot_id, stream=stream)
        for _ in range(steps):
            if w.mode == "one_token":
                ssu.ssu_one_token(state, w.x, w.dt, w.A, w.B, w.C, out,
                                  state_batch_indices=w.src, dst_state_batch_indices=w.dst,
                                  **common)
            else:
                ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, w.cu_seqlens, out,
                                      num_accepted_tokens=w.num_accepted,
                                      state_batch_indices=w.src_table,
                                      dst_state_batch_indices=w.dst_table, **common)

    ref = []
    for w in works:
        state, out = w.state.clone(), w.out_sentinel()
        chain(w, state, out)
        ref.append((state, out))
    torch.cuda.synchronize()

    got = [(w.state.clone(), w.out_sentinel()) for w in works]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in works]
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                chain(works[i], *got[i], stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(works))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for (s_ref, o_ref), (s_got, o_got) in zip(ref, got):
        assert torch.equal(hz.bits(s_ref), hz.bits(s_got))
        assert torch.equal(hz.bits(o_ref), hz.bits(o_got))


# ------------------------------------------------------------- prepared calls

def test_prepared_calls_match_the_regular_calls():
    """A prepared call (checks and marshalling done once) gives the regular
    call's bits, and calling it again continues from the updated state, as two
    regular steps do; one-token, packed and dense forms."""
    import selective_state_update_ssu_amd as ssu
    w = wl.one_token("prep1", 404, batch=9, H=8, P=64, N=128, G=2, nslots=20, device=DEV,
                     pad_fraction=0.2)
    kw = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=True, state_batch_indices=w.src,
              dst_state_batch_indices=w.dst)
    s_reg, s_prep = w.state.clone(), w.state.clone()
    o_reg = torch.full_like(w.x, float("nan"))
    o_prep = torch.full_like(w.x, float("nan"))
    call = ssu.prepare_one_token(s_prep, w.x, w.dt, w.A, w.B, w.C, o_prep, **kw)
    for _ in range(2):
        ssu.ssu_one_token(s_reg, w.x, w.dt, w.A, w.B, w.C, o_reg, **kw)
        assert call() is o_prep
        torch.cuda.synchronize()
        assert torch.equal(hz.bits(o_reg), hz.bits(o_prep))
        assert torch.equal(hz.bits(s_reg), hz.bits(s_prep))

    for dense in (False, True):
        p = wl.packed("prep2", 405, nseq=6, max_len=3, H=4, P=64, N=64, G=1, nslots=40,
                      device=DEV, lengths=None if not dense else [3] * 6, dense=dense)
        pk = dict(num_accepted_tokens=p.num_accepted, state_batch_indices=p.src_table,
                  dst_state_batch_indices=p.dst_table, D=p.D, dt_bias=p.dt_bias,
                  dt_softplus=True)
        s_reg, s_prep = p.state.clone(), p.state.clone()
        if dense:
            d4 = lambda t: None if t is None else t.view(6, 3, *t.shape[1:])
            args = (d4(p.x), d4(p.dt), p.A, d4(p.B), d4(p.C), None)
            pk["z"] = d4(p.z)
        else:
            args = (p.x, p.dt, p.A, p.B, p.C, p.cu_seqlens)
            pk["z"] = p.z
        o_reg = ssu.ssu_packed_varlen(s_reg, *args, **pk)
        call = ssu.prepare_packed_varlen(s_prep, *args, **pk)
        o_prep = call()
        torch.cuda.synchronize()
        assert o_prep.shape == o_reg.shape
        assert torch.equal(hz.bits(o_reg), hz.bits(o_prep)), dense
        assert torch.equal(hz.bits(s_reg), hz.bits(s_prep)), dense


# ------------------------------------------------------- every compiled instance

@pytest.mark.parametrize("mode", ["one_token", "packed"])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_every_compiled_instance(state_dtype, mode):
    """Every (io dtype, dstate, loads per lane) instance of this state dtype and
    entry point -- 30 kernels -- against the oracle on a small ragged shape
    (headdim 72: a partial second row block at every geometry), with pads and
    distinct destinations; and, for a 16-bit state, the stochastically rounding
    instances (bf16 io, every dstate and load depth) against the oracle's
    rounding."""
    n = 0
    for io, N, lpl in itertools.product(["f32", "f16", "bf16"], [16, 32, 64, 128, 256], [2, 4]):
        if mode == "one_token":
            w = wl.one_token("inst", 31, batch=5, H=4, P=72, N=N, G=2, nslots=12, device=DEV,
                             state_dtype=state_dtype, io=io, pad_fraction=0.2,
                             dst_mode="distinct")
        else:
            w = wl.packed("inst", 32, nseq=4, max_len=10, H=4, P=72, N=N, G=2, nslots=48,
                          device=DEV, state_dtype=state_dtype, io=io,
                          lengths=[3, 0, 10, 1], pad_fraction=0.25)
        name = f"{mode}-{state_dtype}-{io}-N{N}-l{lpl}"
        out, after, before = hz.gpu_run(w, loads_per_lane=lpl)
        compare_full(name, w, out, after, before, hz.oracle_full(w))
        n += 1
        if state_dtype != "f32" and io == "bf16":
            w.rand_seed = torch.tensor([0x5EED + N], dtype=torch.int64, device=DEV)
            out, after, before = hz.gpu_run(w, loads_per_lane=lpl)
            hz.check_placement(name + "-sr", w, out, after, before)
            hz.check_slots_sr(name + "-sr state", after, before, list(range(w.state.shape[0])),
                              hz.oracle_full(w).state, hz.oracle_full(w, rounding=False).state)
            n += 1
    _say(f"[parity] every instance, {mode} {state_dtype}: {n} kernels checked")
