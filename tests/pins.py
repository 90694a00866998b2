"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each `pin_*` function takes an `oracle.Oracle` and raises AssertionError when the
oracle disagrees with the fact it checks. `test_oracle_pins.py` runs them on the
real oracle; `test_oracle_mutants.py` runs them on builds of the oracle with a
planted mistake and requires every such build to fail at least one pin.

What pins the oracle (none of these re-types the oracle's loop):
  - scalar cases worked by hand;
  - softplus and sigmoid checked against numpy/scipy library routines;
  - the matrix ("dual", semiseparable) form of the same linear recurrence from
    the Mamba-2 SSD paper (Dao & Gu, ICML 2024), evaluated with numpy matmuls;
  - the zero-decay closed form out_T = sum_{t<=T} dt_t (B_t . C_T) x_t;
  - invariants: dt = 0 keeps the state, superposition, the gate factorises,
    packed = sequential one-token steps, one-token = packed with one token per
    sequence, pad / disable leave memory untouched, the head-to-group map;
  - page examples stored under tests/golden/ (cu_seqlens with an empty sequence,
    regular dense starts, flat-table addressing).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

RTOL = 1e-12


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _softplus(u):
    return np.logaddexp(0.0, u)


def _rand_problem(rng, *, rows, H, P, N, G, nslots, per_dim=False):
    return dict(
        state=rng.standard_normal((nslots, H, P, N)),
        x=rng.standard_normal((rows, H, P)),
        dt=rng.uniform(-3.0, 0.5, (rows, H, P) if per_dim else (rows, H)),
        A=-np.exp(rng.uniform(0.0, 2.0, H)),
        B=rng.standard_normal((rows, G, N)),
        C=rng.standard_normal((rows, G, N)),
        D=rng.standard_normal(H),
        z=rng.standard_normal((rows, H, P)),
        dt_bias=rng.uniform(-1.0, 1.0, H),
    )


# ---------------------------------------------------------------- hand-worked

def pin_scalar_by_hand(orc):
    """H = P = N = G = 1, one slot. s0 = 2, x = 3, dt = 0.5, B = 1, C = 2, D = 1.
    A = 0: dA = 1, s' = 2 + 0.5*1*3 = 3.5, y = 3.5*2 + 1*3 = 10.
    z = 0 gates to 0; z = 2 multiplies by 2*sigmoid(2)."""
    one = np.ones((1, 1, 1))
    kw = dict(x=3 * one, dt=np.array([[0.5]]), B=one, C=2 * one, D=np.array([1.0]))
    r = orc.one_token(np.full((1, 1, 1, 1), 2.0), A=np.array([0.0]), dt_softplus=False, **kw)
    assert r.state[0, 0, 0, 0] == 3.5, r.state
    assert r.out[0, 0, 0] == 10.0, r.out
    r = orc.one_token(np.full((1, 1, 1, 1), 2.0), A=np.array([0.0]), z=0 * one, **kw)
    assert r.out[0, 0, 0] == 0.0, r.out
    r = orc.one_token(np.full((1, 1, 1, 1), 2.0), A=np.array([0.0]), z=2 * one, **kw)
    _close(r.out[0, 0, 0], 10.0 * 2.0 / (1.0 + math.exp(-2.0)), what="gate z=2")
    # A = -1: dA = exp(-0.5); s' = 2 exp(-0.5) + 1.5; y = 2 s' + 3.
    r = orc.one_token(np.full((1, 1, 1, 1), 2.0), A=np.array([-1.0]), **kw)
    s1 = 2.0 * math.exp(-0.5) + 1.5
    _close(r.state[0, 0, 0, 0], s1, what="decay state")
    _close(r.out[0, 0, 0], 2.0 * s1 + 3.0, what="decay out")


def pin_softplus_and_bias(orc):
    """With A = 0, s0 = 0, x = B = 1, C = 1 and no D, y = softplus(dt + dt_bias):
    the output reveals the effective step, which must be numpy's log(1 + e^u)
    of the biased value (bias first, then softplus), or the raw biased value with
    softplus off."""
    u_dt = np.array([-30.0, -4.0, -0.5, 0.0, 0.3, 2.0, 19.0, 25.0, 40.0])
    bias = np.array([0.25])
    n = u_dt.size
    one = np.ones((n, 1, 1))
    for sp in (True, False):
        r = orc.one_token(np.zeros((n, 1, 1, 1)), x=one, dt=u_dt[:, None], A=np.array([0.0]),
                          B=one, C=one, dt_bias=bias, dt_softplus=sp)
        want = _softplus(u_dt + bias[0]) if sp else u_dt + bias[0]
        _close(r.out[:, 0, 0], want, rtol=1e-14, what=f"softplus={sp}")
    # ln 2 at zero; dA = 2^A there.
    r = orc.one_token(np.full((1, 1, 1, 1), 4.0), x=np.zeros((1, 1, 1)), dt=np.array([[0.0]]),
                      A=np.array([-1.0]), B=np.ones((1, 1, 1)), C=np.ones((1, 1, 1)),
                      dt_softplus=True)
    _close(r.state[0, 0, 0, 0], 2.0, rtol=1e-15, what="2^A decay at softplus(0)")


def pin_gate_factorises(orc):
    """out(z) = out(no z) * z * sigmoid(z), with scipy's expit as sigmoid."""
    rng = np.random.default_rng(11)
    pb = _rand_problem(rng, rows=3, H=4, P=8, N=16, G=2, nslots=3)
    z = pb.pop("z")
    a = orc.one_token(dt_softplus=True, **pb)
    b = orc.one_token(dt_softplus=True, z=z, **pb)
    _close(b.out, a.out * z * expit(z), rtol=1e-13, what="gate")
    assert np.array_equal(a.state, b.state)


# ------------------------------------------------------------ independent forms

def _ssd_matrix_form(h0, x, v, A, B, C, D):
    """One head, L tokens: the semiseparable-matrix form of the recurrence.
    h0 [P, N]; x [L, P]; v [L] effective steps; A, D scalars; B, C [L, N].
    Returns y [L, P] and the states after every token [L, P, N]."""
    L = x.shape[0]
    S = np.cumsum(v)
    seg = S[:, None] - S[None, :]                       # S_T - S_t
    decay = np.where(np.tril(np.ones((L, L), dtype=bool)), np.exp(A * np.where(
        np.tril(np.ones((L, L), dtype=bool)), seg, 0.0)), 0.0)
    M = decay * (C @ B.T) * v[None, :]                   # [T, t]
    y = M @ x + np.exp(A * S)[:, None] * (C @ h0.T) + D * x
    states = np.exp(A * S)[:, None, None] * h0[None] + np.einsum(
        "Tt,tp,tn->Tpn", decay * v[None, :], x, B)
    return y, states


def pin_ssd_matrix_form(orc):
    """A packed sequence of L tokens, each writing its own slot, against the
    matrix form of the same recurrence: every intermediate state and output."""
    rng = np.random.default_rng(5)
    L, H, P, N, G = 6, 4, 5, 7, 2
    nslots = L + 1
    pb = _rand_problem(rng, rows=L, H=H, P=P, N=N, G=G, nslots=nslots)
    pb.pop("z")
    table = np.array([[0, 1, 2, 3, 4, 5]])
    dtab = np.array([[6, 1, 2, 3, 4, 5]])      # token t writes slot dtab[t]; token 0 -> slot 6
    r = orc.packed_varlen(cu_seqlens=[0, L], src_table=table, dst_table=dtab,
                          num_accepted=[1], dt_softplus=True, **pb)
    v = _softplus(pb["dt"] + pb["dt_bias"][None, :])     # [L, H]
    hpg = H // G
    for h in range(H):
        g = h // hpg
        y, states = _ssd_matrix_form(pb["state"][0, h], pb["x"][:, h, :], v[:, h], pb["A"][h],
                                     pb["B"][:, g, :], pb["C"][:, g, :], pb["D"][h])
        _close(r.out[:, h, :], y, rtol=1e-11, what=f"y head {h}")
        for t in range(L):
            _close(r.state[dtab[0, t], h], states[t], rtol=1e-11, what=f"state t={t} h={h}")


def pin_zero_decay_closed_form(orc):
    """A = 0, D = 0, no gate, zero initial state:
    out_T[p] = sum_{t<=T} dt_t (B_t . C_T) x_t[p], per head, with per-dim dt."""
    rng = np.random.default_rng(7)
    L, H, P, N, G = 5, 2, 3, 4, 1
    pb = _rand_problem(rng, rows=L, H=H, P=P, N=N, G=G, nslots=1, per_dim=True)
    r = orc.packed_varlen(np.zeros((1, H, P, N)), pb["x"], pb["dt"], np.zeros(H), pb["B"],
                          pb["C"], cu_seqlens=[0, L], dt_softplus=False)
    for h in range(H):
        for T in range(L):
            want = sum(pb["dt"][t, h] * (pb["B"][t, 0] @ pb["C"][T, 0]) * pb["x"][t, h]
                       for t in range(T + 1))
            _close(r.out[T, h], want, rtol=1e-12, what=f"T={T} h={h}")


# ----------------------------------------------------------------- invariants

def pin_zero_step_copies_state(orc):
    """dt + dt_bias = 0 with softplus off: the state is unchanged bit for bit, so
    src != dst copies the slot; out = C . s + D x (numpy dot)."""
    rng = np.random.default_rng(3)
    H, P, N, G, nslots, batch = 4, 6, 8, 2, 8, 3
    pb = _rand_problem(rng, rows=batch, H=H, P=P, N=N, G=G, nslots=nslots)
    pb["dt"] = -np.broadcast_to(pb["dt_bias"], (batch, H)).copy()
    pb.pop("z")
    src, dst = np.array([5, 0, 2]), np.array([1, 7, 3])
    r = orc.one_token(src=src, dst=dst, dt_softplus=False, **pb)
    for b in range(batch):
        assert np.array_equal(r.state[dst[b]], pb["state"][src[b]]), b
        for h in range(H):
            g = h // (H // G)
            want = pb["state"][src[b], h] @ pb["C"][b, g] + pb["D"][h] * pb["x"][b, h]
            _close(r.out[b, h], want, what=f"b={b} h={h}")
    untouched = [s for s in range(nslots) if s not in set(dst.tolist())]
    assert np.array_equal(r.state[untouched], pb["state"][untouched])


def pin_superposition(orc):
    """Without a gate the step is linear in (state, x) jointly."""
    rng = np.random.default_rng(9)
    a = _rand_problem(rng, rows=2, H=3, P=4, N=5, G=1, nslots=2)
    b = _rand_problem(rng, rows=2, H=3, P=4, N=5, G=1, nslots=2)
    for k in ("dt", "A", "B", "C", "D", "dt_bias"):
        b[k] = a[k]
    a.pop("z"), b.pop("z")
    ra = orc.one_token(dt_softplus=True, **a)
    rb = orc.one_token(dt_softplus=True, **b)
    s = dict(a, state=a["state"] + 2.5 * b["state"], x=a["x"] + 2.5 * b["x"])
    rs = orc.one_token(dt_softplus=True, **s)
    _close(rs.out, ra.out + 2.5 * rb.out, rtol=1e-12, what="out")
    _close(rs.state, ra.state + 2.5 * rb.state, rtol=1e-12, what="state")


def pin_packed_equals_sequential(orc):
    """A packed sequence of L tokens equals L one-token calls, call t reading the
    slot call t-1 wrote (or the read slot), bit for bit on an fp64 cache."""
    rng = np.random.default_rng(13)
    H, P, N, G, L = 4, 3, 8, 2, 4
    nslots = 10
    pb = _rand_problem(rng, rows=L, H=H, P=P, N=N, G=G, nslots=nslots)
    table = np.array([[4, 9, 2, 7]])
    r = orc.packed_varlen(cu_seqlens=[0, L], src_table=table, dst_table=table,
                          num_accepted=[3], dt_softplus=True, **pb)
    state = pb["state"].copy()
    read = table[0, 2]
    outs = []
    for t in range(L):
        step = {k: (v[t:t + 1] if k in ("x", "dt", "B", "C", "z") else v)
                for k, v in pb.items() if k != "state"}
        rt = orc.one_token(state, src=[read], dst=[table[0, t]], dt_softplus=True, **step)
        state = rt.state
        outs.append(rt.out[0])
        read = table[0, t]
    assert np.array_equal(r.state, state)
    assert np.array_equal(r.out, np.stack(outs))


def pin_one_token_equals_packed(orc):
    """One token per sequence through the packed form (cu = arange, 1-wide tables)
    equals the one-token form bit for bit; so does the dense [batch, steps] layout
    with regular starts against per-sequence packed calls."""
    rng = np.random.default_rng(17)
    H, P, N, G, batch, nslots = 4, 5, 6, 2, 5, 9
    pb = _rand_problem(rng, rows=batch, H=H, P=P, N=N, G=G, nslots=nslots)
    src = np.array([3, 8, -1, 0, 6])
    dst = np.array([1, 8, 4, 2, -1])
    a = orc.one_token(src=src, dst=dst, dt_softplus=True, **pb)
    b = orc.packed_varlen(cu_seqlens=np.arange(batch + 1), src_table=src[:, None],
                          dst_table=dst[:, None], dt_softplus=True, **pb)
    assert np.array_equal(a.state, b.state)
    assert np.array_equal(a.out, b.out, equal_nan=True)


def pin_pad_and_disable(orc):
    """A pad or out-of-range read slot leaves its out rows and every slot alone; a
    pad destination drops only the write; disabling the update changes no slot
    and no output."""
    rng = np.random.default_rng(19)
    H, P, N, G, nslots = 2, 4, 4, 1, 6
    pb = _rand_problem(rng, rows=5, H=H, P=P, N=N, G=G, nslots=nslots)
    src = np.array([-1, 6, 2, -7, 4])          # pad, out of range, ok, out of range, ok
    dst = np.array([0, 1, -1, 3, 5])           # .., .., pad dst, .., ok
    r = orc.one_token(src=src, dst=dst, dt_softplus=True, **pb)
    for b in (0, 1, 3):
        assert np.all(np.isnan(r.out[b])), b
    assert np.all(np.isfinite(r.out[[2, 4]]))
    changed = [s for s in range(nslots) if not np.array_equal(r.state[s], pb["state"][s])]
    assert changed == [5], changed
    d = orc.one_token(src=src, dst=dst, dt_softplus=True, disable_state_update=True, **pb)
    assert np.array_equal(d.state, pb["state"])
    assert np.array_equal(d.out, r.out, equal_nan=True)
    # A non-default pad id: 2 is now pad, -1 merely out of range.
    q = orc.one_token(src=src, dst=dst, dt_softplus=True, pad_slot_id=2, **pb)
    assert np.all(np.isnan(q.out[2])) and np.all(np.isfinite(q.out[4]))


def pin_group_map(orc):
    """Heads form contiguous blocks of H/G per group: each head of a G-group call
    equals a single-head call fed its group's B/C. G = H with B/C replicated per
    head equals G = 1."""
    rng = np.random.default_rng(23)
    H, P, N, G, batch = 6, 3, 5, 3, 2
    pb = _rand_problem(rng, rows=batch, H=H, P=P, N=N, G=G, nslots=batch)
    full = orc.one_token(dt_softplus=True, **pb)
    for h in range(H):
        g = h // (H // G)
        single = orc.one_token(pb["state"][:, h:h + 1], pb["x"][:, h:h + 1], pb["dt"][:, h:h + 1],
                               pb["A"][h:h + 1], pb["B"][:, g:g + 1], pb["C"][:, g:g + 1],
                               D=pb["D"][h:h + 1], z=pb["z"][:, h:h + 1],
                               dt_bias=pb["dt_bias"][h:h + 1], dt_softplus=True)
        assert np.array_equal(full.out[:, h:h + 1], single.out), h
        assert np.array_equal(full.state[:, h:h + 1], single.state), h
    one = dict(pb, B=pb["B"][:, :1], C=pb["C"][:, :1])
    rep = dict(pb, B=np.repeat(one["B"], H, axis=1), C=np.repeat(one["C"], H, axis=1))
    a = orc.one_token(dt_softplus=True, **one)
    b = orc.one_token(dt_softplus=True, **rep)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.state, b.state)


def pin_accepted_count_selects_entry(orc):
    """With a zero effective step, out = C . s_read + D x names the slot read: it
    must be the table entry k-1; k outside [1, steps] makes the sequence inert."""
    rng = np.random.default_rng(29)
    H, P, N, G, nseq, steps, nslots = 2, 3, 4, 1, 4, 3, 12
    lengths = [1, 2, 3, 2]
    rows = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    pb = _rand_problem(rng, rows=rows, H=H, P=P, N=N, G=G, nslots=nslots)
    pb["dt"] = -np.broadcast_to(pb["dt_bias"], (rows, H)).copy()
    pb.pop("z")
    table = np.arange(nseq * steps).reshape(nseq, steps)
    k = np.array([2, 3, 0, 4])          # two valid, then 0 and steps + 1 (inert)
    r = orc.packed_varlen(cu_seqlens=cu, num_accepted=k, src_table=table, dst_table=table,
                          dt_softplus=False, **pb)
    for b in range(2):
        s = pb["state"][table[b, k[b] - 1]]
        for t in range(lengths[b]):
            row = cu[b] + t
            want = s @ pb["C"][row, 0] + pb["D"][:, None] * pb["x"][row]
            _close(r.out[row], want, what=f"b={b} t={t}")
            assert np.array_equal(r.state[table[b, t]], s)
    for b in (2, 3):
        assert np.all(np.isnan(r.out[cu[b]:cu[b + 1]]))
        for t in range(steps):
            assert np.array_equal(r.state[table[b, t]], pb["state"][table[b, t]])


def pin_missing_destination_writes_back(orc):
    """Without a destination the last token's state lands in the read slot."""
    rng = np.random.default_rng(31)
    H, P, N, G = 2, 2, 3, 1
    pb = _rand_problem(rng, rows=3, H=H, P=P, N=N, G=G, nslots=4)
    table = np.array([[2, 0, 3]])
    a = orc.packed_varlen(cu_seqlens=[0, 3], src_table=table, num_accepted=[2],
                          dt_softplus=True, **pb)
    b = orc.packed_varlen(cu_seqlens=[0, 3], src_table=table, num_accepted=[2],
                          dst_table=np.array([[-1, -1, 0]]), dt_softplus=True, **pb)
    assert np.array_equal(a.state[0], b.state[0])
    assert np.array_equal(a.out, b.out)
    for s in (1, 2, 3):
        assert np.array_equal(a.state[s], pb["state"][s])


# ------------------------------------------------------------- page examples

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_page_examples(orc):
    g = _golden("page_examples.json")
    rng = np.random.default_rng(37)
    H, P, N = 2, 2, 3

    # Query starts [0, 0, 2]: sequence 0 is empty, sequence 1 owns rows 0 and 1.
    ex = g["empty_sequence_starts"]
    cu = np.array(ex["cu_seqlens"])
    rows = int(cu[-1])
    pb = _rand_problem(rng, rows=rows, H=H, P=P, N=N, G=1, nslots=2)
    tab = np.array([[0, 0], [1, 1]])
    r = orc.packed_varlen(cu_seqlens=cu, src_table=tab, dst_table=tab, dt_softplus=True, **pb)
    for b in ex["empty_sequences"]:
        assert np.array_equal(r.state[tab[b, 0]], pb["state"][tab[b, 0]])
    assert list(range(int(cu[1]), int(cu[2]))) == ex["rows_of_sequence_1"]
    seq = orc.packed_varlen(cu_seqlens=[0, rows], src_table=tab[1:], dst_table=tab[1:],
                            dt_softplus=True, **pb)
    assert np.array_equal(r.out, seq.out) and np.array_equal(r.state, seq.state)

    # Dense [batch, steps] layout: starts 0, steps, 2 steps, ... batch * steps.
    ex = g["dense_regular_starts"]
    batch, steps = ex["batch"], ex["steps"]
    starts = np.arange(0, (batch + 1) * steps, steps)
    assert starts.tolist() == ex["cu_seqlens"]
    pb = _rand_problem(rng, rows=batch * steps, H=H, P=P, N=N, G=1, nslots=batch * steps)
    tab = np.arange(batch * steps).reshape(batch, steps)
    dense = orc.packed_varlen(cu_seqlens=starts, src_table=tab, dst_table=tab,
                              dt_softplus=True, **pb)
    for b in range(batch):
        sl = slice(b * steps, (b + 1) * steps)
        one = dict(pb, x=pb["x"][sl], dt=pb["dt"][sl], B=pb["B"][sl], C=pb["C"][sl],
                   z=pb["z"][sl])
        rb = orc.packed_varlen(cu_seqlens=[0, steps], src_table=tab[b:b + 1],
                               dst_table=tab[b:b + 1], dt_softplus=True, **one)
        assert np.array_equal(dense.out[sl], rb.out)
        for t in range(steps):
            assert np.array_equal(dense.state[tab[b, t]], rb.state[tab[b, t]])

    # Flat [rows] table, strides (1, 1): position t of sequence b is entry b + t.
    for ex in g["flat_table_addressing"]["cases"]:
        flat = np.array(ex["table"])
        lengths = ex["lengths"]
        cu = np.concatenate([[0], np.cumsum(lengths)])
        nslots = int(flat.max()) + 1
        pb = _rand_problem(rng, rows=int(cu[-1]), H=H, P=P, N=N, G=1, nslots=nslots)
        r = orc.packed_varlen(cu_seqlens=cu, src_table=flat, src_strides=(1, 1),
                              dst_table=flat, dst_strides=(1, 1), steps=ex["steps"],
                              dt_softplus=True, **pb)
        tab = np.full((len(lengths), ex["steps"]), -1)
        for b, ents in enumerate(ex["entries_written"]):
            for t, e in enumerate(ents):
                tab[b, t] = flat[e]
        r2 = orc.packed_varlen(cu_seqlens=cu, src_table=tab, dst_table=tab,
                               dt_softplus=True, **pb)
        assert np.array_equal(r.out, r2.out) and np.array_equal(r.state, r2.state)
        written = sorted({int(flat[e]) for ents in ex["entries_written"] for e in ents})
        changed = [s for s in range(nslots) if not np.array_equal(r.state[s], pb["state"][s])]
        assert changed == written, (changed, written)


# -------------------------------------------------------------- ring trackers
# The ReplaySSM tracker update / reset and the delayed commit of the vLLM
# `ssu_dispatch` module (its two tracker kernels). Expected values are worked
# by hand from that definition, or closed forms of repeated application.

def _zeros(n):
    return np.zeros(n, dtype=np.int64)


def pin_ring_reset_and_masks(orc):
    """Reset zeroes all three counters of every named valid slot and nothing
    else; pad and out-of-range slots are skipped by update and commit alike; a
    2-D table is addressed through its stride (first column)."""
    rs, pn, pq = np.arange(10, 16), np.arange(20, 26), np.arange(30, 36)
    r = orc.ring_update(rs, pn, pq, [4, -1, 1, 6, 99])
    assert r.ring_start.tolist() == [10, 0, 12, 13, 0, 15]
    assert r.prev_num_accepted.tolist() == [20, 0, 22, 23, 0, 25]
    assert r.prev_query_len.tolist() == [30, 0, 32, 33, 0, 35]
    # A [3, 2] table: entries 0, 2, 4 are the first column.
    table = np.array([[2, 5], [-1, 0], [3, 1]])
    r = orc.ring_update(rs, pn, pq, table, slot_stride=2)
    assert r.ring_start.tolist() == [10, 11, 0, 0, 14, 15]
    a = orc.ring_update(_zeros(4), _zeros(4), _zeros(4), [-1, 7], logical_window=2,
                        ring_buffer_len=4)
    assert a.prev_num_accepted.tolist() == [0, 0, 0, 0]
    c = orc.ring_commit([1, 1, 1, 1], [1, 1, 1, 1], [1, 1, 1, 1], [-1, 9], [3, 3], [0, 2, 5],
                        logical_window=2, ring_buffer_len=4)
    assert c.ring_start.tolist() == [1, 1, 1, 1] and c.prev_query_len.tolist() == [1, 1, 1, 1]


def pin_ring_advance_closed_form(orc):
    """After a reset and K advances with window W >= 1 and ring length R: the
    ring was checkpointed c = floor((K-1)/W) times, each time moving past W
    tokens, so start = (c W) mod R and the count is K - c W. With W = 0 every
    advance checkpoints: start = (K-1) mod R, count 1."""
    for W, R in ((1, 4), (3, 8), (5, 7), (0, 5)):
        r = orc.ring_update(_zeros(3), _zeros(3), _zeros(3), [2])
        for K in range(1, 21):
            r = orc.ring_update(r.ring_start, r.prev_num_accepted, r.prev_query_len, [2],
                                logical_window=W, ring_buffer_len=R)
            if W == 0:
                want = ((K - 1) % R, 1)
            else:
                c = (K - 1) // W
                want = ((c * W) % R, K - c * W)
            got = (int(r.ring_start[2]), int(r.prev_num_accepted[2]))
            assert got == want, (W, R, K, got, want)
            assert r.prev_query_len[2] == 0


def pin_ring_commit_cases(orc):
    """One commit over four slots, each worked by hand (window 6, ring 8):
      slot 0: no previous window (0)     -> count 0, start kept;
      slot 1: 2 counted + window 3 <= 6  -> count 2 + 4 = 6, start kept;
      slot 2: 4 counted + window 3 > 6   -> start 1 + 4 = 5, count = accepted 2;
      slot 3: 5 counted + window 2 > 6   -> start (6 + 5) mod 8 = 3, count 1.
    Each records its current window length from the query starts."""
    rs = [7, 3, 1, 6]
    pn = [9, 2, 4, 5]
    pq = [0, 3, 3, 2]
    slots = [0, 1, 2, 3]
    acc = [5, 4, 2, 1]
    qsl = [0, 2, 5, 9, 10]
    c = orc.ring_commit(rs, pn, pq, slots, acc, qsl, logical_window=6, ring_buffer_len=8)
    assert c.ring_start.tolist() == [7, 3, 5, 3], c
    assert c.prev_num_accepted.tolist() == [0, 6, 2, 1], c
    assert c.prev_query_len.tolist() == [2, 3, 4, 1], c


def pin_ring_commit_sequence(orc):
    """An MTP run on one slot, window 4, ring 16, every query 3 tokens long,
    accepted counts 2, 3, 1, 3, 2 after the first (worked by hand):
    (start, count, window) = (0,0,3) (0,2,3) (2,3,3) (5,1,3) (5,4,3) (9,2,3)."""
    z = _zeros(1)
    r = orc.ring_update(z + 7, z + 7, z + 7, [0])
    want = [(0, 0, 3), (0, 2, 3), (2, 3, 3), (5, 1, 3), (5, 4, 3), (9, 2, 3)]
    for step, acc in enumerate([0, 2, 3, 1, 3, 2]):
        r = orc.ring_commit(r.ring_start, r.prev_num_accepted, r.prev_query_len, [0], [acc],
                            [0, 3], logical_window=4, ring_buffer_len=16)
        got = (int(r.ring_start[0]), int(r.prev_num_accepted[0]), int(r.prev_query_len[0]))
        assert got == want[step], (step, got, want[step])


# -------------------------------------------------------- stochastic rounding

_ROCRAND = {}


def _rocrand_philox(vectors):
    """Philox4x32-10 words from rocRAND's host-callable engine (a library
    routine), for (key0, key1, c0, c1, c2, c3) tuples with c1 < 2^30."""
    import subprocess
    import tempfile
    if "exe" not in _ROCRAND:
        d = tempfile.mkdtemp(prefix="rocrand_philox_")
        exe = os.path.join(d, "rocrand_philox")
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rocrand_philox.cpp")
        subprocess.run(["/opt/rocm/bin/hipcc", "-O1", "--offload-arch=gfx950", "-o", exe, src],
                       check=True, capture_output=True)
        _ROCRAND["exe"] = exe
    text = "".join(" ".join(f"{v:x}" for v in vec) + "\n" for vec in vectors)
    out = subprocess.run([_ROCRAND["exe"]], input=text, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    return [[int(w, 16) for w in line.split()] for line in out if line.strip()]


def pin_philox_matches_rocrand(orc):
    """The oracle's Philox4x32 at 10 rounds equals rocRAND's Philox4x32-10 on
    edge and random keys and counters."""
    rng = np.random.default_rng(41)
    vecs = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF,
                                 0xFFFFFFFF), (1, 0, 7, 3, 0, 0), (0xDEADBEEF, 0, 12345, 0, 1, 0)]
    for _ in range(60):
        k0, k1, c0, c2, c3 = (int(v) for v in rng.integers(0, 2**32, 5))
        vecs.append((k0, k1, c0, int(rng.integers(0, 2**30)), c2, c3))
    ref = _rocrand_philox(vecs)
    for vec, want in zip(vecs, ref):
        got = orc.philox4x32(vec[2:], vec[:2], 10)
        assert got == want, (vec, [hex(g) for g in got], [hex(w) for w in want])


def _fp32_values(rng, n, lo_exp, hi_exp):
    """Random fp32 values with exponents in [lo_exp, hi_exp], both signs."""
    m = rng.integers(0, 2**23, n)
    e = rng.integers(lo_exp, hi_exp + 1, n)
    v = (1.0 + m / 2.0**23) * np.exp2(e)
    v = v.astype(np.float32).astype(np.float64)
    return v * np.where(rng.random(n) < 0.5, -1.0, 1.0)


def pin_stochastic_rounding_is_unbiased(orc):
    """Averaged over the random words, SR returns its input exactly: it rounds
    away from zero with probability equal to the fraction of the spacing the
    value passes. For an fp32 input that fraction has at most b bits (b = 16 for
    bf16, 13 for fp16 normals, 13 + (-14 - e) for fp16 subnormals of exponent e),
    and U >= 1 - frac then depends only on U's top b bits, so the 2^b words whose
    remaining bits are zero give exactly the mean over all words."""
    rng = np.random.default_rng(43)
    cases = [("bf16", 16, _fp32_values(rng, 6, -130, 120)),
             ("f16", 13, _fp32_values(rng, 4, -14, 15)),
             ("f16", 15, _fp32_values(rng, 2, -16, -16)),
             ("f16", 17, _fp32_values(rng, 2, -18, -18)),
             ("f16", 20, _fp32_values(rng, 1, -21, -21))]
    for fmt, b, values in cases:
        words = (np.arange(2**b, dtype=np.uint64) << (32 - b)).astype(np.uint32)
        for v in values:
            r = orc.round_stochastic(np.full(words.shape, v), words, fmt)
            assert np.all(np.isfinite(r))
            assert math.fsum(r) / 2**b == v, (fmt, v, math.fsum(r) / 2**b)


def _format_neighbours(v, fmt):
    """The two values of the format bracketing each v (toward and away from
    zero), from torch's round-to-nearest conversion and the adjacent bit
    patterns (the magnitude bits of a 16-bit float count up by one per value)."""
    import torch
    tdt = torch.bfloat16 if fmt == "bf16" else torch.float16
    n = torch.tensor(v).to(torch.float32).to(tdt)
    nb = n.view(torch.int16).numpy().astype(np.int32)
    nv = n.double().numpy()
    up = torch.tensor((nb + 1).astype(np.int16)).view(tdt).double().numpy()
    dn = torch.tensor(np.maximum(nb - 1, nb & ~0x7FFF).astype(np.int16)).view(tdt).double().numpy()
    toward = np.where(np.abs(nv) <= np.abs(v), nv, dn)
    away = np.where(np.abs(nv) <= np.abs(v), np.where(nv == v, nv, up), nv)
    return toward, away


def pin_stochastic_rounding_neighbours(orc):
    """SR lands on one of the two neighbours of v in the target format, keeps
    representable values, is odd-symmetric, passes 0/inf/nan, and overflows past
    the largest finite value to infinity."""
    rng = np.random.default_rng(47)
    for fmt in ("bf16", "f16"):
        v = _fp32_values(rng, 4000, -20 if fmt == "f16" else -100, 14)
        w = rng.integers(0, 2**32, v.shape[0], dtype=np.uint64).astype(np.uint32)
        r = orc.round_stochastic(v, w, fmt)
        toward, away = _format_neighbours(v, fmt)
        assert np.all((r == toward) | (r == away)), fmt
        assert (r == away).any() and (r == toward).any(), fmt
        rep = toward[:200]
        assert np.array_equal(orc.round_stochastic(rep, w[:200], fmt), rep), fmt
        assert np.array_equal(orc.round_stochastic(-v, w, fmt), -r), fmt
    sp = orc.round_stochastic([0.0, np.inf, -np.inf, np.nan], [0xFFFFFFFF] * 4, "f16")
    assert sp[0] == 0 and sp[1] == np.inf and sp[2] == -np.inf and np.isnan(sp[3])
    assert orc.round_stochastic([65510.0], [0xFFFFFFFF], "f16")[0] == np.inf
    assert orc.round_stochastic([65510.0], [0], "f16")[0] == 65504.0
    bf16_max = (2 - 2.0**-7) * 2.0**127
    big = float(np.float32(3.396e38))            # between bf16's maximum and fp32's
    assert orc.round_stochastic([big], [0xFFFFFFFF], "bf16")[0] == np.inf
    assert orc.round_stochastic([big], [0], "bf16")[0] == bf16_max


def _sr_word(orc, e, row, seed, rounds, fmt):
    """The random word element e of row `row` uses, with its bits at the top:
    fp16 takes word e % 4 of Philox(e / 4, ...); bf16 takes the low (even e) or
    high (odd e) half of word (e % 8) / 2 of Philox(e / 8, ...)."""
    key = [seed & 0xFFFFFFFF, seed >> 32]
    if fmt == "f16":
        return orc.philox4x32([e // 4, row, 0, 0], key, rounds)[e % 4]
    word = orc.philox4x32([e // 8, row, 0, 0], key, rounds)[(e % 8) // 2]
    half = (word >> 16) if e % 2 else (word & 0xFFFF)
    return half << 16


def pin_stochastic_rounding_in_the_update(orc):
    """A stored 16-bit state is SR of the unrounded state with the random bits
    of its element (layout in `_sr_word`; e the element's index within the slot,
    row the token's packed row); rounds as given."""
    rng = np.random.default_rng(53)
    H, P, N, G, L = 2, 3, 8, 1, 3
    pb = _rand_problem(rng, rows=L, H=H, P=P, N=N, G=G, nslots=2 * L)
    table = np.array([[0, 1, 2]])
    dtab = np.array([[3, 4, 5]])
    seed = 0x1234_5678_9ABC_DEF0
    for fmt, rounds in (("bf16", 10), ("f16", 7)):
        plain = orc.packed_varlen(cu_seqlens=[0, L], src_table=table, dst_table=dtab,
                                  dt_softplus=True, **pb)
        sr = orc.packed_varlen(cu_seqlens=[0, L], src_table=table, dst_table=dtab,
                               dt_softplus=True, sr_format=fmt, rand_seed=seed,
                               philox_rounds=rounds, **pb)
        assert np.array_equal(plain.out, sr.out)
        for t in range(L):
            vals = plain.state[dtab[0, t]].reshape(-1)
            words = np.array([_sr_word(orc, e, t, seed, rounds, fmt)
                              for e in range(vals.shape[0])], dtype=np.uint32)
            want = orc.round_stochastic(vals, words, fmt)
            assert np.array_equal(sr.state[dtab[0, t]].reshape(-1), want), (fmt, t)
        for s in range(3):
            assert np.array_equal(sr.state[s], pb["state"][s])


def pin_stochastic_rounding_row_base(orc):
    """A run of consecutive sequences cut out of a call and run with the cut's
    first packed row as the row base stores exactly the bits the whole call
    stores for them (the counters number rows call-wide); without the base the
    bits differ. One-token and packed."""
    rng = np.random.default_rng(59)
    H, P, N, G = 2, 3, 8, 1
    seed, fmt = 0x0F1E_2D3C_4B5A_6978, "bf16"
    # one token per sequence: sequences 3..5 of 7, each writing its own slot
    pb = _rand_problem(rng, rows=7, H=H, P=P, N=N, G=G, nslots=14)
    src, dst = np.arange(7), np.arange(7, 14)
    whole = orc.one_token(src=src, dst=dst, dt_softplus=True, sr_format=fmt, rand_seed=seed,
                          **pb)
    cut = {k: (v[3:6] if k in ("x", "dt", "B", "C", "z") else v) for k, v in pb.items()}
    part = orc.one_token(src=src[3:6], dst=dst[3:6], dt_softplus=True, sr_format=fmt,
                         rand_seed=seed, sr_row_base=3, **cut)
    unbased = orc.one_token(src=src[3:6], dst=dst[3:6], dt_softplus=True, sr_format=fmt,
                            rand_seed=seed, **cut)
    for s_ in dst[3:6]:
        assert np.array_equal(part.state[s_], whole.state[s_]), s_
    assert not all(np.array_equal(unbased.state[s_], whole.state[s_]) for s_ in dst[3:6])
    # packed: sequences 1..2 of lengths [2, 3, 2] own rows 2..6
    pb = _rand_problem(rng, rows=7, H=H, P=P, N=N, G=G, nslots=12)
    table = np.array([[0, 1, 2], [3, 4, 5], [6, 7, 8]])
    whole = orc.packed_varlen(cu_seqlens=[0, 2, 5, 7], src_table=table, dst_table=table,
                              num_accepted=[1, 2, 1], dt_softplus=True, sr_format="f16",
                              rand_seed=seed, **pb)
    cut = {k: (v[2:7] if k in ("x", "dt", "B", "C", "z") else v) for k, v in pb.items()}
    part = orc.packed_varlen(cu_seqlens=[0, 3, 5], src_table=table[1:], dst_table=table[1:],
                             num_accepted=[2, 1], dt_softplus=True, sr_format="f16",
                             rand_seed=seed, sr_row_base=2, **cut)
    for s_ in table[1:].reshape(-1):
        assert np.array_equal(part.state[s_], whole.state[s_]), s_
    assert np.array_equal(part.out, whole.out[2:7])


# ------------------------------------------------------------ SSD prefill

def _ssd_problem(rng, *, lengths, H, P, N, G, chunk, init=True, runs_ids=None):
    """Packed sequences of the given lengths cut into chunks of `chunk` tokens
    (the last chunk of a sequence may be short). Returns the operands and the
    chunk metadata the contract asks for; request ids default to 0, 1, ..."""
    cc, seq_idx, lci = [0], [], []
    ids = list(range(len(lengths))) if runs_ids is None else runs_ids
    for b, L in enumerate(lengths):
        pos = 0
        while True:
            step = min(chunk, L - pos)
            cc.append(cc[-1] + step)
            seq_idx.append(ids[b])
            pos += step
            if pos >= L:
                break
        lci.append(len(seq_idx) - 1)
    T = cc[-1]
    batch = max(ids) + 1
    return dict(
        x=rng.standard_normal((T, H, P)), dt=rng.uniform(-3.0, 0.5, (T, H)),
        A=-np.exp(rng.uniform(0.0, 1.5, H)), B=rng.standard_normal((T, G, N)),
        C=rng.standard_normal((T, G, N)), D=rng.standard_normal(H),
        z=rng.standard_normal((T, H, P)), dt_bias=rng.uniform(-1.0, 1.0, H),
        initial_states=rng.standard_normal((batch, H, P, N)) if init else None,
        chunk_size=chunk, cu_chunk_seqlens=np.array(cc), seq_idx=np.array(seq_idx),
        last_chunk_indices=np.array(lci))


def _ssd_call(orc, pb, **over):
    kw = dict(pb)
    kw.update(over)
    args = [kw.pop(k) for k in ("x", "dt", "A", "B", "C", "chunk_size", "cu_chunk_seqlens",
                                "seq_idx", "last_chunk_indices")]
    return orc.ssd_prefill(*args, **kw)


def _ssd_blocked(pb, dt_softplus, dt_limit=(0.0, np.inf)):
    """The chunked SSD algorithm (the block decomposition of the SSD paper,
    section 6) with numpy matmuls: per chunk, the diagonal block
    (C B^T masked by the decay matrix) applied to v x, the chunk's own state
    from its inputs, the state carried in from the previous chunk of the same
    request, and that state's contribution C h_in scaled by the decay so far."""
    x, dt, A, B, C, D, z = (pb[k] for k in ("x", "dt", "A", "B", "C", "D", "z"))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    ratio = H // G
    v = dt + pb["dt_bias"]
    if dt_softplus:
        v = _softplus(v)
    v = np.clip(v, dt_limit[0], dt_limit[1])
    cc, si = pb["cu_chunk_seqlens"], pb["seq_idx"]
    init = pb["initial_states"]
    out = np.full(x.shape, np.nan)
    states = []
    h_in = None
    for c in range(len(cc) - 1):
        if c == 0 or si[c] != si[c - 1]:
            h_in = init[si[c]].copy() if init is not None else np.zeros((H, P, N))
        lo, hi = cc[c], cc[c + 1]
        L = hi - lo
        if L == 0:
            states.append(h_in.copy())
            continue
        h_out = np.empty_like(h_in)
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(H):
            g = h // ratio
            cum = np.cumsum(A[h] * v[lo:hi, h])                   # decay exponent to t
            seg = np.where(causal, cum[:, None] - cum[None, :], -np.inf)
            Bc, Cc = B[lo:hi, g], C[lo:hi, g]                       # [L, N]
            Xv = x[lo:hi, h] * v[lo:hi, h][:, None]                 # [L, P]
            y = ((Cc @ Bc.T) * np.exp(seg)) @ Xv                    # inside the chunk
            y += np.exp(cum)[:, None] * (Cc @ h_in[h].T)            # from the state in
            own = (Xv * np.exp(cum[-1] - cum)[:, None]).T @ Bc      # [P, N]
            h_out[h] = np.exp(cum[-1]) * h_in[h] + own
            y += D[h] * x[lo:hi, h]
            y *= z[lo:hi, h] * expit(z[lo:hi, h])
            out[lo:hi, h] = y
        h_in = h_out
        states.append(h_out.copy())
    return out, np.stack(states)


def pin_ssd_chunked_form(orc):
    """The SSD prefill equals the chunked (block-decomposed) algorithm of the SSD
    paper, computed with numpy matmuls, for every output and every chunk state:
    three requests of 37, 16 and 5 tokens in chunks of 16, two groups."""
    rng = np.random.default_rng(61)
    pb = _ssd_problem(rng, lengths=[37, 16, 5], H=4, P=3, N=5, G=2, chunk=16)
    r = _ssd_call(orc, pb, dt_softplus=True)
    out, states = _ssd_blocked(pb, True)
    _close(r.out, out, 1e-10, "out")
    _close(r.chunk_states, states, 1e-10, "chunk states")
    assert np.array_equal(r.final_states, r.chunk_states[pb["last_chunk_indices"]])
    # Without initial states every request starts from zero.
    r0 = _ssd_call(orc, pb, dt_softplus=True, initial_states=None)
    out0, states0 = _ssd_blocked(dict(pb, initial_states=None), True)
    _close(r0.out, out0, 1e-10, "out, zero start")
    _close(r0.chunk_states, states0, 1e-10, "states, zero start")


def pin_ssd_equals_decode(orc):
    """Run token by token, a request is the packed decode form over the same
    rows: its output rows agree, and the state after each chunk equals the state
    the decode form stores for that chunk's last token. Requests map to read
    slots holding their initial states; every token writes its own slot."""
    rng = np.random.default_rng(62)
    lengths = [9, 20, 1]
    pb = _ssd_problem(rng, lengths=lengths, H=2, P=3, N=4, G=1, chunk=8)
    r = _ssd_call(orc, pb, dt_softplus=True)
    T = sum(lengths)
    nreq = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    steps = max(lengths)
    dst = np.full((nreq, steps), -1)
    for b in range(nreq):
        dst[b, :lengths[b]] = nreq + cu[b] + np.arange(lengths[b])
    state = np.zeros((nreq + T, 2, 3, 4))
    state[:nreq] = pb["initial_states"]
    d = orc.packed_varlen(state, pb["x"], pb["dt"], pb["A"], pb["B"], pb["C"], cu,
                          src_table=np.arange(nreq)[:, None], dst_table=dst, steps=steps,
                          D=pb["D"], z=pb["z"], dt_bias=pb["dt_bias"], dt_softplus=True)
    _close(r.out, d.out, 1e-12, "out")
    cc = pb["cu_chunk_seqlens"]
    for c in range(len(cc) - 1):
        _close(r.chunk_states[c], d.state[nreq + cc[c + 1] - 1], 1e-12, f"chunk {c}")


def pin_ssd_seq_idx_decides_entering_state(orc):
    """A chunk opens a request when its seq_idx differs from the previous
    chunk's, and then enters with that request's initial state; the returned
    final states are the chunk states the last-chunk indices name, even when
    those indices disagree with seq_idx. Each request, run alone, gives the same
    rows and states bit for bit."""
    rng = np.random.default_rng(63)
    # Requests 2, 0, 1 in that order (ids not in chunk order), 3 chunks, 1 chunk, 2 chunks.
    pb = _ssd_problem(rng, lengths=[20, 7, 12], H=2, P=2, N=3, G=1, chunk=8,
                      runs_ids=[2, 0, 1])
    assert list(pb["seq_idx"]) == [2, 2, 2, 0, 1, 1]
    r = _ssd_call(orc, pb, dt_softplus=True)
    cc = pb["cu_chunk_seqlens"]
    for first, last, rid in ((0, 2, 2), (3, 3, 0), (4, 5, 1)):
        lo, hi = cc[first], cc[last + 1]
        sub = dict(pb, x=pb["x"][lo:hi], dt=pb["dt"][lo:hi], B=pb["B"][lo:hi],
                   C=pb["C"][lo:hi], z=pb["z"][lo:hi],
                   initial_states=pb["initial_states"][rid:rid + 1],
                   cu_chunk_seqlens=cc[first:last + 2] - lo,
                   seq_idx=np.zeros(last - first + 1, dtype=np.int64),
                   last_chunk_indices=np.array([last - first]))
        alone = _ssd_call(orc, sub, dt_softplus=True)
        assert np.array_equal(alone.out, r.out[lo:hi]), rid
        assert np.array_equal(alone.chunk_states, r.chunk_states[first:last + 1]), rid
    odd = _ssd_call(orc, dict(pb, last_chunk_indices=np.array([0, 4, 3])), dt_softplus=True)
    assert np.array_equal(odd.chunk_states, r.chunk_states)
    assert np.array_equal(odd.final_states, r.chunk_states[[0, 4, 3]])


def pin_ssd_dt_limit(orc):
    """The step is clamped to dt_limit after bias and softplus: with softplus off
    and every dt + bias negative, the default lower limit 0 freezes the state
    (out = C . h0 + D x); with A = 0, no D, no gate and a zero start, an upper
    limit u gives out_t = sum_{s<=t} min(v_s, u) (B_s . C_t) x_s over the
    request, and a lower limit raises small steps the same way."""
    rng = np.random.default_rng(64)
    pb = _ssd_problem(rng, lengths=[11, 6], H=2, P=3, N=4, G=1, chunk=4)
    neg = dict(pb, dt=rng.uniform(-3.0, -1.5, pb["dt"].shape), dt_bias=np.full(2, 0.5))
    r = _ssd_call(orc, neg, dt_softplus=False, z=None)
    for b, (first, last) in enumerate(((0, 2), (3, 4))):
        h0 = pb["initial_states"][b]
        lo, hi = pb["cu_chunk_seqlens"][first], pb["cu_chunk_seqlens"][last + 1]
        ref = (np.einsum("tn,hpn->thp", pb["C"][lo:hi, 0], h0)
               + pb["D"][None, :, None] * pb["x"][lo:hi])
        _close(r.out[lo:hi], ref, 1e-12, f"frozen request {b}")
        assert np.array_equal(r.final_states[b], h0)
    for limit in ((0.0, 0.3), (0.6, np.inf)):
        flat = dict(pb, A=np.zeros(2), D=None, z=None, initial_states=None)
        r = _ssd_call(orc, flat, dt_softplus=True, dt_limit=limit)
        v = np.clip(_softplus(pb["dt"] + pb["dt_bias"]), *limit)
        for first, last in ((0, 2), (3, 4)):
            lo, hi = pb["cu_chunk_seqlens"][first], pb["cu_chunk_seqlens"][last + 1]
            for t in range(lo, hi):
                s = np.arange(lo, t + 1)
                bc = pb["B"][s, 0] @ pb["C"][t, 0]                        # [s]
                ref = np.einsum("s,sh,shp->hp", bc, v[s], pb["x"][s])
                _close(r.out[t], ref, 1e-12, f"limit {limit} t={t}")


def pin_ssd_skip_term_per_dim(orc):
    """D given per (head, dim) adds D[h, p] x[t, h, p] before the gate; a [H]
    D equals the [H, P] D with equal columns, bit for bit."""
    rng = np.random.default_rng(65)
    pb = _ssd_problem(rng, lengths=[7, 3], H=3, P=4, N=2, G=1, chunk=4)
    D2 = rng.standard_normal((3, 4))
    with_d = _ssd_call(orc, pb, dt_softplus=True, D=D2, z=None)
    without = _ssd_call(orc, pb, dt_softplus=True, D=None, z=None)
    _close(with_d.out - without.out, D2[None] * pb["x"], 1e-12, "per-dim D")
    per_head = _ssd_call(orc, pb, dt_softplus=True, z=None)
    tied = _ssd_call(orc, pb, dt_softplus=True, z=None,
                     D=np.repeat(pb["D"][:, None], 4, axis=1))
    assert np.array_equal(per_head.out, tied.out)


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
