"""The prefill entry point that allocates nothing (ssu_ssd_prefill_noalloc, the
library's static per-GPU scratch) against ssu_ssd_prefill with a workspace, bit
for bit, on two calls in a row -- the second smaller -- and its allocations: the
binding makes only the returned states."""
import sys

import pytest
import torch

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


def _pair(w):
    """(out, states) of the workspace entry point and of the static-scratch one."""
    import selective_state_update_ssu_amd as ssu
    out_ws = torch.full_like(w.x, float("nan"))
    st_ws = ssu.ssd_combined_fwd_varlen(*w.args(), out=out_ws, **w.kwargs())
    out_st = torch.full_like(w.x, float("nan"))
    st_st = ssu.ssd_combined_fwd_varlen(*w.args(), out=out_st, static_scratch=True,
                                        **w.kwargs())
    torch.cuda.synchronize()
    return (out_ws, st_ws), (out_st, st_st)


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_static_scratch_matches_workspace_entry():
    first = wl.ssd("noalloc_a", 71, lengths=[1, 255, 256, 257, 700, 37], H=4, P=64, N=128, G=2,
                   chunk=256, device=DEV, with_init=True)
    second = wl.ssd("noalloc_b", 72, lengths=[130, 5, 128], H=2, P=64, N=64, G=1, chunk=128,
                    device=DEV, io="f16", state_dtype="bf16")
    for w in (first, second):
        _say(f"[no-alloc] {w.name}: tokens {w.x.shape[0]}, chunks {w.seq_idx.numel()}")
        (o1, s1), (o2, s2) = _pair(w)
        assert torch.equal(_bits(o1), _bits(o2)), w.name
        assert torch.equal(_bits(s1), _bits(s2)), w.name
        _say(f"[no-alloc] {w.name}: static scratch equals the workspace call bit for bit")


def test_static_scratch_allocates_only_the_states():
    import selective_state_update_ssu_amd as ssu
    w = wl.ssd("noalloc_c", 73, lengths=[300, 40], H=4, P=64, N=128, G=2, chunk=128, device=DEV,
               with_init=True)
    out = torch.empty_like(w.x)
    ssu.ssd_combined_fwd_varlen(*w.args(), out=out, static_scratch=True, **w.kwargs())
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    states = ssu.ssd_combined_fwd_varlen(*w.args(), out=out, static_scratch=True, **w.kwargs())
    made = torch.cuda.memory_stats()["allocation.all.allocated"] - before
    torch.cuda.synchronize()
    assert made == 1, made
    assert torch.isfinite(states.float()).all()


def test_static_scratch_too_small_raises():
    """A call whose workspace exceeds the static scratch is refused on the host."""
    import selective_state_update_ssu_amd as ssu
    w = wl.ssd("noalloc_big", 74, lengths=[35 * 128], H=128, P=64, N=128, G=8, chunk=128,
               device=DEV, with_z=False)
    with pytest.raises(NotImplementedError, match="static scratch holds"):
        ssu.ssd_combined_fwd_varlen(*w.args(), static_scratch=True, **w.kwargs())
