"""SSD chunked prefill on the GPU against the fp64 oracle, element by element:
16-bit results within 1e-2 + 2e-2 |ref|, fp32 states within 1e-5 of their scale
(ssd_harness.py)."""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle
import ssd_harness as sh
from selective_state_update_ssu_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


CASES = {
    # bf16 io, fp32 states, ragged requests (1, Q-1, Q, Q+1, several chunks), two
    # groups, initial states, gate.
    "bf16_f32_ragged": dict(lengths=[1, 255, 256, 257, 700, 37], H=4, P=64, N=128, G=2,
                            chunk=256, with_init=True),
    "bf16_f32_all_chunks": dict(lengths=[1, 255, 256, 257, 700, 37], H=4, P=64, N=128, G=2,
                                chunk=256, with_init=True, return_intermediate_states=True),
    # fp16 io, bf16 states, dstate 64, chunk 128, no initial states, no gate,
    # per-dim D, bf16 dt.
    "f16_bf16_d64": dict(lengths=[130, 5, 128, 300], H=6, P=64, N=64, G=3, chunk=128,
                         io="f16", state_dtype="bf16", with_z=False, D_per_dim=True,
                         dt_dtype="bf16"),
    # fp16 states with a dt limit and softplus off (clamped from below).
    "bf16_f16_limit": dict(lengths=[77, 400, 129], H=2, P=64, N=128, G=1, chunk=128,
                           state_dtype="f16", with_init=True, dt_softplus=False,
                           dt_range=(-1.0, 1.5), dt_limit=(0.05, 0.8)),
    # one long request: fourteen chunks passed from state to state; int64 metadata.
    "f16_f32_long": dict(lengths=[3500], H=2, P=64, N=64, G=1, chunk=256, io="f16",
                         with_init=True, meta_dtype="i64", return_intermediate_states=True),
    # request ids out of chunk order; fp16 dt.
    "ids_out_of_order": dict(lengths=[300, 40, 520], H=4, P=64, N=128, G=4, chunk=128,
                             with_init=True, request_ids=[2, 0, 1], dt_dtype="f16"),
    # more runs of chunks than the state walk ranks by length (2048): they are
    # walked in chunk order; a few multi-chunk requests among 2100.
    "more_runs_than_ranked": dict(lengths=[1 + (7 * i) % 5 for i in range(2096)]
                                  + [300, 700, 129, 257], H=2, P=64, N=64, G=1, chunk=128,
                                  with_init=True),
    # headdim 128 (two 64-column blocks in the walk and the scan); bf16 io, fp32
    # states, chunk 256, ragged requests, initial states, gate.
    "headdim128": dict(lengths=[1, 255, 300, 700], H=4, P=128, N=128, G=2, chunk=256,
                       with_init=True),
    # headdim 128 with fp16 io, bf16 states, dstate 64, chunk 128, every chunk's state.
    "headdim128_f16_all_chunks": dict(lengths=[130, 5, 400], H=2, P=128, N=64, G=1, chunk=128,
                                      io="f16", state_dtype="bf16",
                                      return_intermediate_states=True),
    # dstate 256 (two 128-row blocks in the walk, eight k steps in the scan).
    "dstate256": dict(lengths=[37, 256, 600], H=4, P=64, N=256, G=2, chunk=256, with_init=True),
    "dstate256_q128_f16_states": dict(lengths=[129, 700, 3], H=2, P=64, N=256, G=1, chunk=128,
                                      state_dtype="f16", with_init=True, D_per_dim=True),
    # both at once, and headdim 192 and 256
    "headdim128_dstate256": dict(lengths=[300, 90], H=2, P=128, N=256, G=1, chunk=128,
                                 with_init=True, return_intermediate_states=True),
    "headdim192": dict(lengths=[200, 333], H=2, P=192, N=128, G=1, chunk=256, with_init=True),
    "headdim256_f16": dict(lengths=[150, 260], H=2, P=256, N=64, G=2, chunk=128, io="f16",
                           with_init=True, D_per_dim=True),
    # chunks of 128 take two heads per scan workgroup: an odd head count leaves
    # the last workgroup of each chunk one head, and one group per head puts
    # the two heads of a workgroup in different groups; two column blocks.
    "odd_heads_q128": dict(lengths=[200, 129, 7], H=5, P=128, N=128, G=5, chunk=128,
                           with_init=True, D_per_dim=True),
}


def _make(name, seed=5):
    kw = dict(CASES[name])
    extra = {k: kw.pop(k) for k in ("return_intermediate_states", "dt_softplus", "dt_limit")
             if k in kw}
    return wl.ssd(name, seed, device=DEV, **kw, **extra)


@pytest.mark.parametrize("name", sorted(CASES))
def test_small_cases(name):
    w = _make(name)
    print(f"[ssd] {name}: tokens {w.x.shape[0]}, chunks {w.seq_idx.numel()}", flush=True)
    out = torch.full_like(w.x, float("nan"))
    _, states = sh.run_gpu(w, out)
    torch.cuda.synchronize()
    ref, mag = sh.oracle_ref(w)
    (r_out, d_out), (r_st, d_st) = sh.check_all(w, out, states, ref, mag)
    print(f"[ssd] {name}: worst err/bar out {r_out:.3f}, states {r_st:.3f} "
          f"(diagnostic err/terms: out {d_out:.3f}, states {d_st:.3f})", flush=True)


def test_last_chunk_indices_disagreeing_with_seq_idx():
    """The returned per-request states are the chunk states the last-chunk
    indices name, even when those disagree with seq_idx; seq_idx alone decides
    where each chunk's entering state comes from."""
    w = _make("bf16_f32_ragged")
    nchunks = w.seq_idx.numel()
    w.last_chunk_indices = torch.tensor([0, 3, 3, nchunks - 1, 1, 2], dtype=torch.int32,
                                        device=DEV)
    out = torch.empty_like(w.x)
    _, states = sh.run_gpu(w, out)
    torch.cuda.synchronize()
    ref, mag = sh.oracle_ref(w)
    sh.check_all(w, out, states, ref, mag)


def test_out_allocated_when_absent_and_written_in_place():
    import selective_state_update_ssu_amd as ssu
    w = _make("f16_bf16_d64")
    states = ssu.ssd_combined_fwd_varlen(*w.args(), **w.kwargs())
    out = torch.empty_like(w.x)
    states2 = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())
    torch.cuda.synchronize()
    assert torch.equal(states, states2)
    ref, mag = sh.oracle_ref(w)
    sh.check_out(out, ref.out, mag.out, w.x.dtype)


def test_repeatable_bit_for_bit():
    w = _make("bf16_f32_ragged")
    a = torch.empty_like(w.x)
    b = torch.empty_like(w.x)
    _, sa = sh.run_gpu(w, a)
    _, sb = sh.run_gpu(w, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)


@pytest.mark.parametrize("name", ["ssd_mamba2_2p7b", "ssd_nemotron_h"])
def test_named_workload_every_request(name):
    """The full-size prefill, as the benchmark runs it; every request is cut out
    (all heads) and checked against the oracle on every row of out and on its
    final state. The oracle runs the requests on parallel host threads."""
    from concurrent.futures import ThreadPoolExecutor
    w = wl.SSD_NAMED[name](DEV)
    print(f"[ssd] {name}: tokens {w.x.shape[0]}, chunks {w.seq_idx.numel()}", flush=True)
    out = torch.full_like(w.x, float("nan"))
    _, states = sh.run_gpu(w, out)
    torch.cuda.synchronize()
    nreq = len(w.meta["lengths"])
    cuts = [sh.cut_request(w, b) for b in range(nreq)]
    orc = oracle.default()
    with ThreadPoolExecutor(max_workers=min(16, nreq, os.cpu_count() or 1)) as ex:
        refs = list(ex.map(lambda cut: sh.oracle_ref(cut[0], orc), cuts))
    worst = [0.0, 0.0]
    for b, ((cut, (lo, hi), hs), (ref, mag)) in enumerate(zip(cuts, refs)):
        (r_out, d_out) = sh.check_out(out[lo:hi], ref.out, mag.out, w.x.dtype,
                                      what=f"out of request {b}")
        (r_st, d_st) = sh.check_states(states[b:b + 1], ref.final_states, mag.final_states,
                                       w.state_dtype, w.x.dtype, f"state of request {b}")
        worst = [max(worst[0], r_out), max(worst[1], r_st)]
        print(f"[ssd] {name} request {b} ({hi - lo} tokens): worst err/bar out {r_out:.3f}, "
              f"state {r_st:.3f} (diagnostic {d_out:.3f}, {d_st:.3f})", flush=True)
    print(f"[ssd] {name}: {nreq} of {nreq} requests compared, all heads; worst err/bar "
          f"out {worst[0]:.3f}, states {worst[1]:.3f}", flush=True)


def test_empty_request_list_and_chunks():
    """No requests to return (batch 0) and an empty chunk: the call still runs and
    writes the rows of the chunks it has."""
    import selective_state_update_ssu_amd as ssu
    w = _make("bf16_f32_all_chunks")
    cc = w.cu_chunk_seqlens.cpu().tolist()
    # Append an empty chunk of a new request 6 (no initial state row for it: the
    # states come back per chunk, so batch stays as it was).
    w.cu_chunk_seqlens = torch.tensor(cc + [cc[-1]], dtype=torch.int32, device=DEV)
    w.seq_idx = torch.cat([w.seq_idx, torch.tensor([5], dtype=torch.int32, device=DEV)])
    out = torch.empty_like(w.x)
    _, states = sh.run_gpu(w, out)
    torch.cuda.synchronize()
    ref, mag = sh.oracle_ref(w)
    sh.check_all(w, out, states, ref, mag)
    # Without initial states and with return_intermediate_states the batch may be 0.
    states = ssu.ssd_combined_fwd_varlen(
        w.x, w.dt, w.A, w.B, w.C, w.chunk_size, w.cu_seqlens[:1], w.cu_chunk_seqlens,
        w.last_chunk_indices[:0], w.seq_idx, out=out, D=w.D, z=w.z, dt_bias=w.dt_bias,
        dt_softplus=True, return_intermediate_states=True, state_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.default().ssd_prefill(
        *(sh.np64(t) for t in (w.x, w.dt, w.A, w.B, w.C)), w.chunk_size,
        sh.npi(w.cu_chunk_seqlens), sh.npi(w.seq_idx), np.zeros(0, dtype=np.int64),
        D=sh.np64(w.D), z=sh.np64(w.z), dt_bias=sh.np64(w.dt_bias), dt_softplus=True)
    w.initial_states = None
    _, mag = sh.oracle_ref(w)
    sh.check_states(states, ref.chunk_states, mag.chunk_states, torch.float32, w.x.dtype)


def test_repeated_calls_allocate_only_the_returned_states():
    """After the first call of a shape, each further call on the same stream
    makes exactly one allocation (the returned states): the workspace is cached.
    A caller-provided workspace gives the same bits; reset drops the cache."""
    import selective_state_update_ssu_amd as ssu
    w = _make("bf16_f32_ragged")
    out = torch.empty_like(w.x)
    first = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())
    torch.cuda.synchronize()
    counts = []
    for _ in range(3):
        before = torch.cuda.memory_stats()["allocation.all.allocated"]
        states = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())
        counts.append(torch.cuda.memory_stats()["allocation.all.allocated"] - before)
        assert torch.equal(states, first)
        del states
    print(f"[ssd] allocations per repeated call: {counts}", flush=True)
    assert counts == [1, 1, 1], counts
    nchunks, batch = w.seq_idx.numel(), w.last_chunk_indices.numel()
    H, P, N, G = w.x.shape[1], w.x.shape[2], w.B.shape[2], w.B.shape[1]
    ws = torch.empty(ssu.ssd_workspace_bytes(nchunks, batch, H, P, N, G, w.chunk_size),
                     dtype=torch.uint8, device=DEV)
    out2 = torch.empty_like(w.x)
    mine = ssu.ssd_combined_fwd_varlen(*w.args(), out=out2, workspace=ws, **w.kwargs())
    torch.cuda.synchronize()
    assert torch.equal(mine, first) and torch.equal(out2, out)
    with pytest.raises(ValueError):
        ssu.ssd_combined_fwd_varlen(*w.args(), out=out2, workspace=ws[:100], **w.kwargs())
    ssu.reset_ssd_workspaces()
    assert ssu._ssd_workspaces == {}


def test_explicit_stream():
    """A prefill on a side stream given as `stream`: the same bits as on the
    current stream, and its workspace is that stream's own."""
    import selective_state_update_ssu_amd as ssu
    w = _make("f16_bf16_d64")
    out = torch.empty_like(w.x)
    ref_states = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out2 = torch.empty_like(w.x)
    side.wait_stream(torch.cuda.current_stream())
    states = ssu.ssd_combined_fwd_varlen(*w.args(), out=out2, stream=side, **w.kwargs())
    side.synchronize()
    assert torch.equal(states, ref_states) and torch.equal(out2, out)
    keys = {k[1] for k in ssu._ssd_workspaces}
    assert side.cuda_stream in keys


def test_two_threads_on_two_streams():
    """Two host threads, each with a stream of its own, repeat prefills of
    different shapes at once: every result equals the single-threaded one bit
    for bit (each stream gets its own cached workspace)."""
    import threading
    import selective_state_update_ssu_amd as ssu
    ws = [_make("bf16_f32_ragged"), _make("ids_out_of_order")]
    refs = []
    for w in ws:
        out = torch.empty_like(w.x)
        refs.append((out, ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())))
    torch.cuda.synchronize()
    results = [[], []]
    errors = []

    def worker(i):
        try:
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                for _ in range(6):
                    out = torch.empty_like(ws[i].x)
                    st = ssu.ssd_combined_fwd_varlen(*ws[i].args(), out=out, **ws[i].kwargs())
                    results[i].append((out, st))
            side.synchronize()
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 6
        for out, st in results[i]:
            assert torch.equal(out, refs[i][0]) and torch.equal(st, refs[i][1]), i


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_every_compiled_instance(io):
    """Every compiled prefill instance of this io type -- state dtype x dstate
    64/128/256 x chunk 128/256, 18 kernel sets -- against the oracle at the
    bars on a small case: two requests (one of a single chunk, one of three with
    a ragged tail), headdim 128, two groups, initial states, gate."""
    worst = [0.0, 0.0]
    n = 0
    for st, N, Q in itertools.product(["f32", "f16", "bf16"], [64, 128, 256], [128, 256]):
        w = wl.ssd(f"inst_{io}_{st}_{N}_{Q}", 41, device=DEV, lengths=[Q - 3, 2 * Q + 37], H=4,
                   P=128, N=N, G=2, chunk=Q, io=io, state_dtype=st, with_init=True)
        out = torch.full_like(w.x, float("nan"))
        _, states = sh.run_gpu(w, out)
        torch.cuda.synchronize()
        ref, mag = sh.oracle_ref(w)
        (r_out, _), (r_st, _) = sh.check_all(w, out, states, ref, mag)
        worst = [max(worst[0], r_out), max(worst[1], r_st)]
        n += 1
    print(f"[ssd] every instance, {io} io: {n} kernel sets, worst err/bar out {worst[0]:.3f}, "
          f"states {worst[1]:.3f}", flush=True)
