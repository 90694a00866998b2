"""Graph capture. The one-token and packed decode steps and the SSD prefill are
recorded into a HIP graph (torch.cuda.CUDAGraph, which captures the stream the
binding launches on) and replayed several times, with unrelated eager work and
a synchronisation between replays. Every replay must equal the same number of
eager calls bit for bit: the kernels and their inputs are the same, and none of
the calls allocates, copies between host and device or synchronises."""
import pytest
import torch

import selective_state_update_ssu_amd as ssu
from selective_state_update_ssu_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 4


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _decode_call(w, state, out):
    common = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                  pad_slot_id=w.pad_slot_id)
    if w.mode == "one_token":
        return lambda: ssu.ssu_one_token(state, w.x, w.dt, w.A, w.B, w.C, out,
                                         state_batch_indices=w.src,
                                         dst_state_batch_indices=w.dst, **common)
    return lambda: ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, w.cu_seqlens, out,
                                         num_accepted_tokens=w.num_accepted,
                                         state_batch_indices=w.src_table,
                                         dst_state_batch_indices=w.dst_table, **common)


def _same_bits(a, b):
    """Bit-for-bit equality (NaN sentinels of untouched rows included)."""
    view = {2: torch.int16, 4: torch.int32}[a.element_size()]
    return torch.equal(a.view(view), b.view(view))


def _busy(n=1 << 20):
    """Unrelated eager work between replays."""
    a = torch.randn(n, device=DEV)
    return float((a * 2 + 1).sum())


@pytest.mark.parametrize("make", [
    lambda: wl.one_token("graph_one_token", 21, batch=64, H=8, P=64, N=128, G=2, nslots=128,
                         device=DEV, pad_fraction=0.1),
    lambda: wl.packed("graph_packed", 22, nseq=32, max_len=4, H=8, P=64, N=128, G=1,
                      nslots=256, device=DEV, pad_fraction=0.1),
], ids=["one_token", "packed"])
def test_decode_graph_replays_match_eager(make):
    """The step updates the state in place, so replay i must equal eager call i."""
    w = make()
    s_eager, s_graph = w.state.clone(), w.state.clone()
    o_eager, o_graph = w.out_sentinel(), w.out_sentinel()
    eager = _decode_call(w, s_eager, o_eager)
    eager()  # loads the library before capture; the graph side starts one step later
    _decode_call(w, s_graph, o_graph)()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_call(w, s_graph, o_graph)()
    for i in range(REPLAYS):
        eager()
        g.replay()
        _busy()
        torch.cuda.synchronize()
        assert _same_bits(o_graph, o_eager), f"replay {i}: out differs from the eager call"
        assert _same_bits(s_graph, s_eager), f"replay {i}: state differs from the eager call"


def test_ssd_prefill_graph_replays_match_eager():
    w = wl.ssd("graph_ssd", 23, lengths=[300, 5, 700, 129], H=8, P=64, N=128, G=2, chunk=256,
               device=DEV, with_init=True)
    o_eager = torch.empty_like(w.x)
    st_eager = ssu.ssd_combined_fwd_varlen(*w.args(), out=o_eager, **w.kwargs())
    torch.cuda.synchronize()
    o_graph = torch.full_like(w.x, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st_graph = ssu.ssd_combined_fwd_varlen(*w.args(), out=o_graph, **w.kwargs())
    for i in range(REPLAYS):
        o_graph.fill_(float("nan"))
        g.replay()
        _busy()
        torch.cuda.synchronize()
        assert _same_bits(o_graph, o_eager), f"replay {i}: out differs from the eager call"
        assert _same_bits(st_graph, st_eager), f"replay {i}: states differ from the eager call"
