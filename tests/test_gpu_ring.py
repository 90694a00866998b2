"""ReplaySSM ring-tracker kernels on the GPU against the oracle, exactly."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_update_ssu_amd as ssu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _trackers(rng, num_states, window, ring, dtype):
    rs = rng.integers(0, ring, num_states)
    pn = rng.integers(0, window + 3, num_states)
    pq = rng.integers(0, 6, num_states) * (rng.random(num_states) < 0.8)
    return [torch.tensor(a, dtype=dtype, device=DEV) for a in (rs, pn, pq)]


def _slots(rng, n, num_states, dtype, table_width=None):
    """n distinct positions: mostly valid slots, some pad (-1), some beyond the
    trackers; optionally as the first column of an [n, width] table."""
    s = rng.permutation(num_states + 64)[:n]
    s[rng.random(n) < 0.1] = -1
    if table_width:
        t = np.full((n, table_width), 12345)
        t[:, 0] = s
        s = t
    return torch.tensor(s, dtype=dtype, device=DEV)


def _check(gpu_trackers, ref):
    got = [t.cpu().numpy().astype(np.int64) for t in gpu_trackers]
    for name, g, r in zip(("ring_start", "prev_num_accepted", "prev_query_len"), got,
                          (ref.ring_start, ref.prev_num_accepted, ref.prev_query_len)):
        assert np.array_equal(g, r), (name, np.nonzero(g != r)[0][:10])


@pytest.mark.parametrize("tdt,sdt,width", [(torch.int32, torch.int32, None),
                                           (torch.int64, torch.int64, None),
                                           (torch.int32, torch.int64, 4)])
def test_reset_advance_commit(tdt, sdt, width):
    rng = np.random.default_rng(11)
    orc = oracle.default()
    num_states, n, W, R = 3000, 700, 5, 13
    trk = _trackers(rng, num_states, W, R, tdt)
    slots = _slots(rng, n, num_states, sdt, width)
    stride = width or 1
    host = [t.cpu().numpy() for t in trk]
    s_host = slots.cpu().numpy().reshape(-1)

    ssu.update_replayssm_ring_trackers(*trk, slots, logical_window=W, ring_buffer_len=R)
    ref = orc.ring_update(*host, s_host, logical_window=W, ring_buffer_len=R,
                          slot_stride=stride, n=n)
    torch.cuda.synchronize()
    _check(trk, ref)

    acc = torch.tensor(rng.integers(0, 6, n), dtype=tdt, device=DEV)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(rng.integers(1, 5, n))]), dtype=tdt,
                       device=DEV)
    ssu.commit_replayssm_ring_trackers(*trk, slots, acc, qsl, W, R)
    ref = orc.ring_commit(ref.ring_start, ref.prev_num_accepted, ref.prev_query_len, s_host,
                          acc.cpu().numpy(), qsl.cpu().numpy(), logical_window=W,
                          ring_buffer_len=R, slot_stride=stride, n=n)
    torch.cuda.synchronize()
    _check(trk, ref)

    ssu.reset_replayssm_ring_trackers(*trk, slots)
    ref = orc.ring_update(ref.ring_start, ref.prev_num_accepted, ref.prev_query_len, s_host,
                          slot_stride=stride, n=n)
    torch.cuda.synchronize()
    _check(trk, ref)


def test_mtp_run_many_steps():
    """Twenty rounds of an MTP decode loop (commit, then a few advances) on 256
    sequences, compared after every call."""
    rng = np.random.default_rng(12)
    orc = oracle.default()
    num_states, n, W, R = 512, 256, 6, 32
    trk = [torch.zeros(num_states, dtype=torch.int32, device=DEV) for _ in range(3)]
    slots = _slots(rng, n, num_states, torch.int32)
    s_host = slots.cpu().numpy()
    ssu.reset_replayssm_ring_trackers(*trk, slots)
    ref = orc.ring_update(*[t.cpu().numpy() for t in trk], s_host)
    for step in range(20):
        acc = torch.tensor(rng.integers(1, 4, n), dtype=torch.int32, device=DEV)
        qsl = torch.tensor(np.concatenate([[0], np.cumsum(rng.integers(1, 5, n))]),
                           dtype=torch.int32, device=DEV)
        ssu.commit_replayssm_ring_trackers(*trk, slots, acc, qsl, W, R)
        ref = orc.ring_commit(ref.ring_start, ref.prev_num_accepted, ref.prev_query_len,
                              s_host, acc.cpu().numpy(), qsl.cpu().numpy(), logical_window=W,
                              ring_buffer_len=R)
        for _ in range(step % 3):
            ssu.update_replayssm_ring_trackers(*trk, slots, logical_window=W, ring_buffer_len=R)
            ref = orc.ring_update(ref.ring_start, ref.prev_num_accepted, ref.prev_query_len,
                                  s_host, logical_window=W, ring_buffer_len=R)
        torch.cuda.synchronize()
        _check(trk, ref)


def test_large_and_empty():
    rng = np.random.default_rng(13)
    orc = oracle.default()
    num_states, n = 1 << 20, 600_000
    trk = _trackers(rng, num_states, 8, 64, torch.int32)
    slots = _slots(rng, n, num_states, torch.int64)
    host = [t.cpu().numpy() for t in trk]
    ssu.update_replayssm_ring_trackers(*trk, slots, logical_window=8, ring_buffer_len=64)
    ref = orc.ring_update(*host, slots.cpu().numpy(), logical_window=8, ring_buffer_len=64)
    torch.cuda.synchronize()
    _check(trk, ref)
    empty = slots[:0]
    ssu.update_replayssm_ring_trackers(*trk, empty, logical_window=8, ring_buffer_len=64)
    torch.cuda.synchronize()
    _check(trk, ref)
