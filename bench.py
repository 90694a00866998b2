#!/usr/bin/env python3
"""SSU decode throughput on one MI355X: tokens/s and achieved HBM GB/s.

A step is one call of the update over one synthetic decode batch with every
input already resident in HBM. The headline workload is the largest decode
configuration, the Nemotron-H-shaped one-token batch (512 sequences, 128 heads x
64 x 128, 8 groups, fp32 state in 1024 slots, bf16 x/B/C/z). The other named
workloads are timed too and reported under "workloads", each with its own
roofline block. The roofline figure divides the algorithmic bytes of one launch
by the launch's average duration from HIP events on the launch stream.

No timed point can be served from the 256 MB Infinity Cache: a workload whose
call touches less than 1 GiB of state cycles through enough copies of its state
cache that at least 1 GiB of state lies between two uses of one copy.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode full|kernel|copy]

--mode kernel times only the chosen workload (for profiler runs; an ssd_* name
times the SSD chunked prefill; --record PATH writes its JSON record there);
--mode copy times only the reference copy kernel used to calibrate traffic
counters; --mode sweep times the one-token step over decode batch sizes (back to
back and replayed from a HIP graph) and over dstate and state widths, one JSON
line per point. The SSD prefill workloads are reported under "workloads" with
their own oracle baseline.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSU tokens/sec and achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
HEADLINE = "nemotron_h"
# Bytes of state that must lie between two uses of one state copy (4x the
# 256 MB Infinity Cache).
MIN_TOUCH_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--mode", choices=["full", "kernel", "copy", "summarize", "sweep"],
                    default="full")
    ap.add_argument("--prof-dir", help="summarize: directory holding the rocprofv3 passes")
    ap.add_argument("--prof-cmd", default="", help="summarize: the command lines that made them")
    ap.add_argument("--heads-per-block", type=int, default=0)
    ap.add_argument("--loads-per-lane", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=6.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--record", help="kernel mode: also write the JSON record to this file")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "selective_state_update_ssu_amd", "csrc", "ssu_*")))
    files.append(os.path.join(ROOT, "include", "ssu.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# ----------------------------------------------------------------- accounting

def _np(t):
    return None if t is None else t.detach().cpu().numpy().astype("int64")


def accounting(w):
    """Live rows, and the bytes the method must move for one call: every live
    sequence reads its state once and writes it once per valid destination;
    live rows read x (and z, dt, B, C) and write out. Inert sequences and
    dropped writes move nothing."""
    import numpy as np

    nslots, H, P, N, G = w.dims
    ssz = w.state.element_size()
    iosz = w.x.element_size()
    pad = w.pad_slot_id

    def ok(s):
        return s != pad and 0 <= s < nslots

    live_seqs = live_rows = writes = 0
    if w.mode == "one_token":
        src = _np(w.src) if w.src is not None else np.arange(w.rows)
        dst = _np(w.dst) if w.dst is not None else src
        for b in range(w.rows):
            if ok(int(src[b])):
                live_seqs += 1
                live_rows += 1
                writes += int(ok(int(dst[b])) and not w.disable_state_update)
        index_bytes = w.rows * 4 * (1 + (w.dst is not None))
    else:
        cu = _np(w.cu_seqlens)
        st, dt_ = _np(w.src_table), _np(w.dst_table)
        na = _np(w.num_accepted)
        steps = st.shape[1] if st is not None else (dt_.shape[1] if dt_ is not None else 1)
        for b in range(len(cu) - 1):
            lo, hi = int(cu[b]), int(cu[b + 1])
            if lo < 0 or hi > w.rows or hi <= lo:
                continue
            k = int(na[b]) if na is not None else 1
            if st is not None and not 1 <= k <= steps:
                continue
            r = int(st[b, k - 1]) if st is not None else b
            if not ok(r):
                continue
            live_seqs += 1
            live_rows += hi - lo
            if w.disable_state_update:
                continue
            if dt_ is None:
                writes += 1
            else:
                writes += sum(ok(int(dt_[b, t])) for t in range(min(hi - lo, steps)))
        index_bytes = (len(cu) + len(cu) - 1) * 4 + 2 * w.rows * 4
    slot_head = H * P * N * ssz
    dt_cols = w.dt.shape[2] if w.dt.dim() == 3 else 1
    row_bytes = H * P * iosz * (2 + (w.z is not None)) + 2 * G * N * iosz + 4 * H * dt_cols
    state_read = live_seqs * slot_head
    state_write = writes * slot_head
    out_bytes = live_rows * H * P * iosz
    total = state_read + state_write + live_rows * row_bytes + index_bytes + 3 * 4 * H
    write = state_write + out_bytes
    return dict(live_rows=live_rows, live_seqs=live_seqs, state_writes=writes,
                state_read_bytes=state_read, state_write_bytes=state_write,
                read_bytes=total - write, write_bytes=write, bytes=total)


# ---------------------------------------------------------------------- timing

def make_call(w, hpb, lpl=0, order=0, state=None):
    import torch
    import selective_state_update_ssu_amd as ssu

    state = w.state if state is None else state
    out = torch.empty_like(w.x)
    common = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                  pad_slot_id=w.pad_slot_id, disable_state_update=w.disable_state_update,
                  rand_seed=w.rand_seed, philox_rounds=w.philox_rounds,
                  heads_per_block=hpb, loads_per_lane=lpl, tile_order=order)
    if w.mode == "one_token":
        return lambda: ssu.ssu_one_token(state, w.x, w.dt, w.A, w.B, w.C, out,
                                         state_batch_indices=w.src,
                                         dst_state_batch_indices=w.dst, **common)
    if w.meta.get("dense"):
        nseq = w.cu_seqlens.shape[0] - 1
        d4 = lambda t: None if t is None else t.view(nseq, -1, *t.shape[1:])
        x4, dt4, B4, C4, out4 = d4(w.x), d4(w.dt), d4(w.B), d4(w.C), d4(out)
        common["z"] = d4(w.z)
        return lambda: ssu.ssu_packed_varlen(state, x4, dt4, w.A, B4, C4, None, out4,
                                             num_accepted_tokens=w.num_accepted,
                                             state_batch_indices=w.src_table,
                                             dst_state_batch_indices=w.dst_table, **common)
    return lambda: ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, w.cu_seqlens, out,
                                         num_accepted_tokens=w.num_accepted,
                                         state_batch_indices=w.src_table,
                                         dst_state_batch_indices=w.dst_table, **common)


def time_calls(call, steps, warmup):
    """Warm up, then time exactly `steps` calls. `call` is one callable or a list
    cycled through (call i runs calls[i % len]). Returns (wall ms per step, event
    ms per launch on the launch stream)."""
    import torch

    calls = call if isinstance(call, (list, tuple)) else [call]
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        calls[i % len(calls)]()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, start.elapsed_time(end) / steps


def state_copies(acc):
    """Copies of the state cache to cycle through so that at least
    MIN_TOUCH_BYTES of state lie between two uses of one copy."""
    touched = acc["state_read_bytes"] + acc["state_write_bytes"]
    return max(1, -(-MIN_TOUCH_BYTES // max(touched, 1)))


def prepared_calls(w, copies=1):
    """Prepared one-token calls (checks and marshalling done once) on `copies`
    copies of the state cache."""
    import torch
    import selective_state_update_ssu_amd as ssu

    out = torch.empty_like(w.x)
    states = [w.state] + [w.state.clone() for _ in range(copies - 1)]
    return [ssu.prepare_one_token(st, w.x, w.dt, w.A, w.B, w.C, out, D=w.D, z=w.z,
                                  dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                                  state_batch_indices=w.src, dst_state_batch_indices=w.dst)
            for st in states]


def rotated_calls(w, hpb, lpl=0, copies=1):
    """`copies` calls of the workload, each on its own copy of the state cache
    (the first on w.state itself)."""
    states = [w.state] + [w.state.clone() for _ in range(copies - 1)]
    return [make_call(w, hpb, lpl, state=st) for st in states]


def stream_library():
    import ctypes
    from selective_state_update_ssu_amd import build
    lib = ctypes.CDLL(build.STREAM_LIBRARY)
    lib.ssu_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
    lib.ssu_stream_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.ssu_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.ssu_stream_fanout.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    return lib


def pattern_ceiling(w, steps, warmup):
    """Launch time of the packed call's state traffic alone (each live sequence's
    tiles read once from the read slot and written to every valid destination,
    no arithmetic) on the workload's own tensors, or None where the streaming
    kernel does not apply (one-token calls, separate read and write tables, head
    tiles not a multiple of 8 KiB)."""
    import torch

    if w.mode != "packed" or w.src_table is None or w.src_table is not w.dst_table:
        return None
    nslots, H, P, N = w.state.shape
    head_bytes = P * N * w.state.element_size()
    if H % 4 or head_bytes % 8192:
        return None
    table = w.src_table.to(torch.int32).contiguous()
    nseq = table.shape[0]
    acc = (w.num_accepted if w.num_accepted is not None
           else torch.ones(nseq, device=table.device)).to(torch.int32).contiguous()
    starts = w.cu_seqlens.to(torch.int32).contiguous()
    lib = stream_library()
    s = torch.cuda.current_stream().cuda_stream
    call = lambda: lib.ssu_stream_fanout(w.state.data_ptr(), nslots, H, head_bytes,
                                         table.data_ptr(), table.shape[1], acc.data_ptr(),
                                         starts.data_ptr(), nseq, s)
    if call() != 0:
        raise RuntimeError("ssu_stream_fanout failed")
    _, ev = time_calls(call, steps, warmup)
    return ev * 1e3


def ceilings(steps=30, nbytes=2 << 30, kinds=("copy", "read", "write")):
    """HBM GB/s of plain streaming kernels over `nbytes` buffers: a copy (bytes
    read plus bytes written), a read-only and a write-only pass."""
    import torch

    lib = stream_library()
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    calls = {
        "copy": (lambda: lib.ssu_stream_copy(b.data_ptr(), a.data_ptr(), nbytes, s), 2 * nbytes),
        "read": (lambda: lib.ssu_stream_read(a.data_ptr(), nbytes, sink.data_ptr(), s), nbytes),
        "write": (lambda: lib.ssu_stream_write(b.data_ptr(), nbytes, s), nbytes),
    }
    out = {}
    for k in kinds:
        call, moved = calls[k]
        _, ev = time_calls(call, steps, 3)
        out[k] = moved / (ev * 1e-3) / 1e9
    return out


def traffic_for(workload, kernel_ms):
    """HBM bytes per launch measured by FETCH_SIZE / WRITE_SIZE (scaled by the
    copy-kernel calibration), if the counters were taken on the current kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def ring_tracker_times(steps=200):
    """Launch time of the ReplaySSM ring-tracker advance and commit kernels for a
    decode batch (256 slots) and a large one (65536), int32 counters."""
    import torch
    import selective_state_update_ssu_amd as ssu

    out = {}
    for n in (256, 65536):
        num_states = 2 * n
        g = torch.Generator(device="cuda")
        g.manual_seed(n)
        trk = [torch.zeros(num_states, dtype=torch.int32, device="cuda") for _ in range(3)]
        slots = torch.randperm(num_states, generator=g, device="cuda")[:n].to(torch.int32)
        acc = torch.ones(n, dtype=torch.int32, device="cuda")
        qsl = torch.arange(0, 2 * n + 1, 2, dtype=torch.int32, device="cuda")
        _, adv = time_calls(lambda: ssu.update_replayssm_ring_trackers(
            *trk, slots, logical_window=8, ring_buffer_len=64), steps, 10)
        _, com = time_calls(lambda: ssu.commit_replayssm_ring_trackers(
            *trk, slots, acc, qsl, 8, 64), steps, 10)
        out[f"n{n}"] = {"advance_us": adv * 1e3, "commit_us": com * 1e3}
    return out


# ------------------------------------------------------------------ CPU leg

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_threads():
    """Host threads for the CPU leg: every CPU this process may run on, capped by
    OMP_NUM_THREADS when the environment sets it (a host shared by several GPUs
    may grant each GPU's jobs a share of its CPUs, and say so there)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else max(1, n)


def cpu_baseline(seconds, name=HEADLINE, nseq=32, block=32):
    """The fp64 oracle on a bounded sample of the headline workload -- its first
    `nseq` sequences, from the same draw the GPU timed, copied to the host -- split
    into independent (block of `block` sequences, head) tasks, each an oracle call
    on that head's state rows, x, dt, z and its group's B and C. First one thread
    runs the tasks in turn for about `seconds`, then one thread per available core
    does (each thread its own tasks, round robin); the oracle releases the
    interpreter lock inside its C calls, so they run in parallel and nothing in
    the oracle changes. Rates are tokens/s: (sequence, head) units done / heads /
    wall time."""
    import threading
    import numpy as np
    import torch
    import oracle
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.NAMED[name]("cuda")
    nslots, H, P, N, G = w.dims
    hpg = H // G
    src_all = w.src.long().cpu().numpy()
    src = src_all[:nseq]
    used = sorted(set(int(v) for v in src))
    remap = {v: i for i, v in enumerate(used)}
    f64 = lambda t: t.detach().double().cpu().numpy()
    state = f64(w.state[torch.as_tensor(used, device=w.state.device)])  # [slots, H, P, N]
    x, dt, z = f64(w.x[:nseq]), f64(w.dt[:nseq]), f64(w.z[:nseq]) if w.z is not None else None
    B, C = f64(w.B[:nseq]), f64(w.C[:nseq])
    A, D, bias = f64(w.A), f64(w.D), f64(w.dt_bias)
    del w
    torch.cuda.empty_cache()
    tasks = []
    for b0 in range(0, nseq, block):
        r = slice(b0, b0 + block)
        s_loc = np.array([remap[int(v)] for v in src[r]])
        rows = sorted(set(s_loc.tolist()))
        rmap = {v: i for i, v in enumerate(rows)}
        sl = np.array([rmap[v] for v in s_loc])
        for h in range(H):
            g = h // hpg
            tasks.append(dict(
                state=np.ascontiguousarray(state[rows][:, h:h + 1]),
                x=np.ascontiguousarray(x[r, h:h + 1]), dt=np.ascontiguousarray(dt[r, h:h + 1]),
                A=A[h:h + 1], B=np.ascontiguousarray(B[r, g:g + 1]),
                C=np.ascontiguousarray(C[r, g:g + 1]), D=D[h:h + 1],
                z=None if z is None else np.ascontiguousarray(z[r, h:h + 1]),
                dt_bias=bias[h:h + 1], src=sl, units=len(sl)))
    orc = oracle.default()

    def run(mine, out, i):
        units = 0
        t0 = time.perf_counter()
        k = 0
        while True:
            t = mine[k % len(mine)]
            orc.one_token(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                          z=t["z"], dt_bias=t["dt_bias"], dt_softplus=True, src=t["src"],
                          dst=t["src"])
            units += t["units"]
            k += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        out[i] = (units, el)

    one = [None]
    run(tasks, one, 0)
    single = one[0][0] / H / one[0][1]
    threads = min(cpu_threads(), len(tasks))
    res = [None] * threads
    ts = [threading.Thread(target=run, args=(tasks[i::threads], res, i)) for i in range(threads)]
    t0 = time.perf_counter()
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    wall = time.perf_counter() - t0
    units = sum(u for u, _ in res)
    try:
        available = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        available = os.cpu_count()
    return {"value": units / H / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread_value": single, "host_cpus": os.cpu_count(),
            "available_cpus": available, "cpu_model": cpu_model(),
            "sample": f"the first {nseq} of the {name} batch's {len(src_all)} sequences (same draw as the "
                      f"GPU run; {H} heads, their slots), as {len(tasks)} ({block}-sequence block, "
                      f"head) oracle calls in fp64; {threads} threads for {wall:.1f} s did "
                      f"{units} (sequence, head) units = {units / H:.0f} tokens; one thread: "
                      f"{single:.0f} tokens/s"}


def torch_index(idx):
    import torch
    return torch.as_tensor(idx, dtype=torch.long)


# ------------------------------------------------------------ profile summary

def readable_kernel_name(mangled):
    """ssu_update_kernel<state, io, dstate, loads per lane, packed, stochastic>
    from the mangled name (the template arguments of this one kernel)."""
    import re
    m = re.match(r"_ZN3ssu17ssu_update_kernelI(.*)EEvNS_12KernelParamsE$", mangled)
    if not m:
        return mangled
    types = {"f": "float", "DF16_": "_Float16", "DF16b": "__bf16"}
    args, rest = [], m.group(1)
    while rest:
        for code, name in types.items():
            if rest.startswith(code):
                args.append(name)
                rest = rest[len(code):]
                break
        else:
            lit = re.match(r"L([ib])(\d+)E", rest)
            if not lit:
                return mangled
            args.append(("true" if lit.group(2) == "1" else "false") if lit.group(1) == "b"
                         else lit.group(2))
            rest = rest[lit.end():]
    return f"ssu_update_kernel<{', '.join(args)}>"


def _csv_rows(pattern):
    import csv
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize(prof_dir, workload, cmd):
    """Summarise rocprofv3 output under prof_dir: kt/ (kernel trace + stats),
    pmc_FETCH_SIZE/ and pmc_WRITE_SIZE/ (SSU kernel), cal_FETCH_SIZE/ and
    cal_WRITE_SIZE/ (the streaming copy of 2 GiB each way). Writes the summary
    to profiles/ and records the calibrated traffic in profiles/traffic.json."""
    import statistics
    from selective_state_update_ssu_amd import workloads as wl

    stats = [r for r in _csv_rows(os.path.join(prof_dir, "kt", "**", "*kernel_stats.csv"))
             if "ssu_update_kernel" in r["Name"]]
    if len(stats) != 1:
        raise SystemExit(f"expected one SSU kernel in the stats, found {len(stats)}")
    kname, avg_ns = stats[0]["Name"], float(stats[0]["AverageNs"])

    def counter(sub, name, kernel_pred):
        vals = [float(r["Counter_Value"]) for r in
                _csv_rows(os.path.join(prof_dir, sub, "**", "*counter_collection.csv"))
                if r["Counter_Name"] == name and kernel_pred(r["Kernel_Name"])]
        return (statistics.median(vals) if vals else None), len(vals)

    is_ssu = lambda n: "ssu_update_kernel" in n
    is_copy = lambda n: "copy_kernel" in n
    fetch_kib, nf = counter("pmc_FETCH_SIZE", "FETCH_SIZE", is_ssu)
    write_kib, nw = counter("pmc_WRITE_SIZE", "WRITE_SIZE", is_ssu)
    cal_fetch, _ = counter("cal_FETCH_SIZE", "FETCH_SIZE", is_copy)
    cal_write, _ = counter("cal_WRITE_SIZE", "WRITE_SIZE", is_copy)
    copy_bytes = 2 << 30
    f_fetch = copy_bytes / (cal_fetch * 1024)
    f_write = copy_bytes / (cal_write * 1024)
    read_b = fetch_kib * 1024 * f_fetch
    write_b = write_kib * 1024 * f_write
    w = wl.NAMED[workload]("cpu")
    acc = accounting(w)
    traffic = read_b + write_b
    algo_read, algo_write = acc["read_bytes"], acc["write_bytes"]
    gbps = acc["bytes"] / (avg_ns * 1e-9) / 1e9
    short = readable_kernel_name(kname)
    md = f"""# {short} on {workload}

Kernel: `{kname}`

Commands (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):
```
{cmd.strip()}
```

| quantity | value |
|---|---|
| average kernel duration (kernel trace, {stats[0]['Calls']} calls) | {avg_ns / 1e3:.1f} us |
| algorithmic bytes per launch | {acc['bytes'] / 1e6:.2f} MB (read {algo_read / 1e6:.2f}, write {algo_write / 1e6:.2f}) |
| algorithmic bandwidth at that duration | {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.3f} of 8 TB/s) |
| FETCH_SIZE per dispatch (median of {nf}) | {fetch_kib:.1f} KiB |
| WRITE_SIZE per dispatch (median of {nw}) | {write_kib:.1f} KiB |
| copy calibration, 2 GiB each way: FETCH_SIZE / WRITE_SIZE | {cal_fetch:.1f} / {cal_write:.1f} KiB |
| scale factors (true bytes / counter bytes) | fetch {f_fetch:.4f}, write {f_write:.4f} |
| calibrated HBM traffic per launch | {traffic / 1e6:.2f} MB (read {read_b / 1e6:.2f}, write {write_b / 1e6:.2f}) |
| traffic / algorithmic bytes | {traffic / acc['bytes']:.4f} |
"""
    occ = {n: counter("pmc_OCC", n, is_ssu) for n in ("OccupancyPercent", "MeanOccupancyPerActiveCU")}
    if all(v[1] for v in occ.values()):
        md += (f"| occupancy, % of the waves a CU can hold (median of {occ['OccupancyPercent'][1]}) "
               f"| {occ['OccupancyPercent'][0]:.1f} % |\n"
               f"| MeanOccupancyPerActiveCU (rocprofv3 derived counter) | "
               f"{occ['MeanOccupancyPerActiveCU'][0]:.1f} |\n")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out_md = os.path.join(ROOT, "profiles", f"ssu_update_kernel_{workload}.md")
    with open(out_md, "w") as f:
        f.write(md)
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        rec = {"kernel_source_sha256": kernel_source_hash(), "workloads": {}}
    rec["workloads"][workload] = {
        "kernel": kname, "avg_ns": avg_ns, "fetch_kib": fetch_kib, "write_kib": write_kib,
        "fetch_scale": f_fetch, "write_scale": f_write, "hbm_bytes_per_launch": traffic,
        "algorithmic_bytes": acc["bytes"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(md)


# ------------------------------------------------------------- SSD prefill

def ssd_accounting(w):
    """Algorithmic bytes and flops of one SSD prefill call. Bytes: every input
    read once (x, z, B, C, dt, initial states, per-head parameters, chunk
    metadata), out and the returned states written once. Flops: the products of
    the chunked algorithm -- C B^T over each chunk's lower triangle per group,
    each chunk's own state, the intra-chunk product and the entering-state
    product -- at 2 flops per multiply-add."""
    import numpy as np
    T, H, P = w.x.shape
    G, N = w.B.shape[1], w.B.shape[2]
    io = w.x.element_size()
    ssz = {"torch.float32": 4}.get(str(w.state_dtype), 2)
    cc = w.cu_chunk_seqlens.cpu().numpy().astype(np.int64)
    si = w.seq_idx.cpu().numpy().astype(np.int64)
    L = np.diff(cc)
    nchunks = L.shape[0]
    batch = w.last_chunk_indices.numel()
    opens = np.ones(nchunks, dtype=bool)
    opens[1:] = si[1:] != si[:-1]
    entering = ~opens | (w.initial_states is not None)
    rows_out = nchunks if w.return_intermediate_states else batch
    meta = (w.cu_chunk_seqlens.numel() + 2 * nchunks + batch) * w.cu_chunk_seqlens.element_size()
    read = (T * H * P * io * (1 + (w.z is not None)) + 2 * T * G * N * io
            + T * H * w.dt.element_size() + 3 * 4 * H + meta
            + (batch * H * P * N * ssz if w.initial_states is not None else 0))
    write = T * H * P * io + rows_out * H * P * N * ssz
    pairs = L * (L + 1) // 2
    flops = float(np.sum(2 * pairs * N * G) + np.sum(2 * L) * H * P * N
                  + np.sum(2 * pairs) * H * P + np.sum(2 * L[entering]) * H * P * N)
    return dict(tokens=T, read_bytes=read, write_bytes=write, bytes=read + write, flops=flops,
                nchunks=nchunks, batch=batch)


def ssd_call(w):
    import torch
    import selective_state_update_ssu_amd as ssu
    out = torch.empty_like(w.x)
    return lambda: ssu.ssd_combined_fwd_varlen(*w.args(), out=out, **w.kwargs())


def run_ssd_workload(name, steps, warmup):
    import torch
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.SSD_NAMED[name]("cuda")
    acc = ssd_accounting(w)
    wall, ev = time_calls(ssd_call(w), steps, warmup)
    T, H, P = w.x.shape
    rec = dict(config=dict(workload=name, mode="ssd_prefill", tokens=T,
                           requests=acc["batch"], chunks=acc["nchunks"], chunk_size=w.chunk_size,
                           nheads=H, headdim=P, dstate=w.B.shape[2], ngroups=w.B.shape[1],
                           io_dtype=str(w.x.dtype).replace("torch.", ""),
                           state_dtype=str(w.state_dtype).replace("torch.", ""),
                           initial_states=w.initial_states is not None, gate=w.z is not None),
               us_per_prefill=ev * 1e3, ms_per_step=wall, tokens_per_s=T / (wall * 1e-3),
               hbm_gbps=acc["bytes"] / (ev * 1e-3) / 1e9,
               tflops=acc["flops"] / (ev * 1e-3) / 1e12, bytes=acc["bytes"], flops=acc["flops"])
    rec["frac_of_peak"] = rec["hbm_gbps"] / HBM_PEAK_GBPS
    del w
    torch.cuda.empty_cache()
    return rec


def ssd_cpu_baseline(seconds):
    """The fp64 oracle on the first request of the Mamba2-2.7B-shaped prefill,
    repeated for about `seconds`: half of the time one thread on all heads
    (`single_thread_value`), half one thread per available core, each task an
    oracle call on a block of heads (the shape has one group, so every block
    reads the same B and C; a head's recurrence needs nothing from another)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.ssd_mamba2_2p7b("cpu")
    H = w.x.shape[1]
    assert w.B.shape[1] == 1, "head blocks share the single group"
    cc = w.cu_chunk_seqlens.numpy().astype(np.int64)
    si = w.seq_idx.numpy().astype(np.int64)
    chunks = np.nonzero(si == 0)[0]
    hi = int(cc[chunks[-1] + 1])
    meta = (w.chunk_size, cc[:chunks[-1] + 2], np.zeros(len(chunks), dtype=np.int64),
            np.array([len(chunks) - 1]))

    def task(h0, h1):
        f = lambda t: np.ascontiguousarray(t[:hi, h0:h1].double().numpy())
        g = lambda t: np.ascontiguousarray(t[h0:h1].double().numpy())
        args = (f(w.x), f(w.dt), g(w.A), w.B[:hi].double().numpy(), w.C[:hi].double().numpy(),
                *meta)
        kw = dict(D=g(w.D), z=f(w.z), dt_bias=g(w.dt_bias), dt_softplus=True)
        return args, kw

    orc = oracle.default()

    def run(tasks, threads, budget):
        """(sequence, head) units per second: every task repeatedly, `threads` at a time."""
        done = 0
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            while time.perf_counter() - t0 < budget:
                heads = list(ex.map(lambda t: (orc.ssd_prefill(*t[1][0], **t[1][1]), t[0])[1],
                                    tasks))
                done += sum(heads)
        return done / (time.perf_counter() - t0)

    whole = [(H, task(0, H))]
    one = run(whole, 1, seconds / 2) * hi / H
    threads = cpu_threads()
    per = -(-H // threads)
    blocks = [(min(h0 + per, H) - h0, task(h0, min(h0 + per, H))) for h0 in range(0, H, per)]
    many = run(blocks, threads, seconds / 2) * hi / H
    return {"value": many, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread_value": one, "cpu_model": cpu_model(),
            "sample": f"request 0 of ssd_mamba2_2p7b ({hi} tokens, {H} heads), fp64: one "
                      f"thread on all heads for {seconds / 2:.1f} s, then {threads} threads "
                      f"on {len(blocks)} blocks of up to {per} heads for {seconds / 2:.1f} s"}


def summarize_ssd(prof_dir, workload, cmd):
    """Per-kernel summary of the SSD prefill under prof_dir: kt/ (kernel trace and
    stats) and, when present, pmc_FETCH_SIZE/, pmc_WRITE_SIZE/ with the copy
    calibration cal_FETCH_SIZE/, cal_WRITE_SIZE/. Writes profiles/ssd_prefill_<workload>.md."""
    import statistics
    from selective_state_update_ssu_amd import workloads as wl

    stats = [r for r in _csv_rows(os.path.join(prof_dir, "kt", "**", "*kernel_stats.csv"))
             if "ssd" in r["Name"]]
    if not stats:
        raise SystemExit("no SSD kernels in the stats")
    order = ["ssd_front_kernel", "ssd_state_walk_kernel", "ssd_scan_kernel"]
    short = lambda n: next((k for k in order if k in n), n)

    def counter(sub, name, pred):
        vals = [float(r["Counter_Value"]) for r in
                _csv_rows(os.path.join(prof_dir, sub, "**", "*counter_collection.csv"))
                if r["Counter_Name"] == name and pred(r["Kernel_Name"])]
        return statistics.median(vals) if vals else None

    have_pmc = os.path.isdir(os.path.join(prof_dir, "pmc_FETCH_SIZE"))
    if have_pmc:
        copy = lambda n: "copy_kernel" in n
        f_fetch = (2 << 30) / (counter("cal_FETCH_SIZE", "FETCH_SIZE", copy) * 1024)
        f_write = (2 << 30) / (counter("cal_WRITE_SIZE", "WRITE_SIZE", copy) * 1024)
    w = wl.SSD_NAMED[workload]("cpu")
    acc = ssd_accounting(w)
    lines, total = [], 0.0
    for r in sorted(stats, key=lambda r: order.index(short(r["Name"]))
                    if short(r["Name"]) in order else 99):
        k = short(r["Name"])
        us = float(r["AverageNs"]) / 1e3
        total += us
        traffic = ""
        if have_pmc:
            pred = lambda n, k=k: k in n
            fk = counter("pmc_FETCH_SIZE", "FETCH_SIZE", pred)
            wk = counter("pmc_WRITE_SIZE", "WRITE_SIZE", pred)
            if fk is not None and wk is not None:
                rb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
                traffic = (f"{rb / 1e6:.1f} | {wb / 1e6:.1f} | "
                           f"{(rb + wb) / (us * 1e-6) / 1e9:.0f}")
        util = counter("pmc_MFMA", "MfmaUtil", lambda n, k=k: k in n)
        occ = counter("pmc_OCC", "OccupancyPercent", lambda n, k=k: k in n)
        extra = (f" {util:.1f} |" if util is not None else " - |") + \
                (f" {occ:.1f} |" if occ is not None else " - |")
        lines.append(f"| `{k}` | {r['Calls']} | {us:.1f} | {traffic or '- | - | -'} |{extra}")
    T = acc["tokens"]
    md = f"""# SSD prefill on {workload}

{T} tokens in {acc['nchunks']} chunks of at most {w.chunk_size} ({acc['batch']} requests),
{w.x.shape[1]} heads x {w.x.shape[2]} x dstate {w.B.shape[2]}, {w.B.shape[1]} groups.

Commands (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):
```
{cmd.strip()}
```

| kernel | calls | average duration (us) | HBM read (MB) | HBM write (MB) | HBM GB/s | MFMA busy % | occupancy % |
|---|---|---|---|---|---|---|---|
{chr(10).join(lines)}

| quantity | value |
|---|---|
| sum of average kernel durations per prefill | {total:.1f} us |
| tokens/s at that time | {T / (total * 1e-6) / 1e6:.2f} M |
| algorithmic bytes per prefill | {acc['bytes'] / 1e6:.1f} MB (read {acc['read_bytes'] / 1e6:.1f}, write {acc['write_bytes'] / 1e6:.1f}) |
| algorithmic bandwidth | {acc['bytes'] / (total * 1e-6) / 1e9:.0f} GB/s ({acc['bytes'] / (total * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of 8 TB/s) |
| flops of the chunked products per prefill | {acc['flops'] / 1e9:.1f} GFLOP ({acc['flops'] / (total * 1e-6) / 1e12:.1f} TFLOP/s) |
"""
    out_md = os.path.join(ROOT, "profiles", f"ssd_prefill_{workload}.md")
    with open(out_md, "w") as f:
        f.write(md)
    print(md)


# ---------------------------------------------------------------------- main

def describe(w):
    nslots, H, P, N, G = w.dims
    d = dict(workload=w.name, mode=w.mode, rows=w.rows, nheads=H, headdim=P, dstate=N,
             ngroups=G, nslots=nslots, state_dtype=str(w.state.dtype).replace("torch.", ""),
             io_dtype=str(w.x.dtype).replace("torch.", ""), gate=w.z is not None,
             disable_state_update=w.disable_state_update)
    if w.mode == "packed":
        d["nseq"] = int(w.cu_seqlens.shape[0] - 1)
    return d


def roofline_block(name, acc, kernel_us):
    gbps = acc["bytes"] / (kernel_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic_for(name, kernel_us * 1e-3),
            "algorithmic_bytes": acc["bytes"], "kernel_us": kernel_us}


def run_workload(name, steps, warmup, hpb, lpl=0):
    import torch
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.NAMED[name]("cuda")
    acc = accounting(w)
    copies = state_copies(acc)
    cache_resident = copies > 64
    if cache_resident:
        # A launch-bound call whose state is a few hundred KB: it stays in the
        # caches whatever we do; its figure is not an HBM one.
        copies = 1
    wall, ev = time_calls(rotated_calls(w, hpb, lpl, copies), steps, warmup)
    rec = dict(config=describe(w), ms_per_step=wall, kernel_us=ev * 1e3,
               tokens_per_s=acc["live_rows"] / (wall * 1e-3),
               hbm_gbps=acc["bytes"] / (ev * 1e-3) / 1e9, state_copies=copies, **acc)
    rec["frac_of_peak"] = rec["hbm_gbps"] / HBM_PEAK_GBPS
    rec["roofline"] = roofline_block(name, acc, rec["kernel_us"])
    if cache_resident:
        rec["cache_resident"] = True
    pattern_us = pattern_ceiling(w, steps, warmup)
    if pattern_us is not None:
        # The same state reads and writes with no arithmetic: how close the
        # kernel comes to pure data movement of its own access pattern.
        rec["state_traffic_only_us"] = pattern_us
        rec["frac_of_state_traffic_only"] = pattern_us / rec["kernel_us"]
    del w
    torch.cuda.empty_cache()
    return rec


def sweep(steps, warmup):
    """One-token calls of the Mamba2-2.7B head shape (80 heads x 64 rows, bf16 io
    with gate, default launch shape): (1) fp32 state, dstate 128, batch 1 ..
    1024, timed back to back (regular and prepared calls) and as `steps` calls
    captured in one HIP graph (the graph shows the device time where the host
    bounds the eager rate);
    (2) dstate 16 .. 256 with fp32 and bf16 state, batch chosen for ~1.35 GB
    per call. Prints one JSON line per point."""
    import statistics
    import torch
    from selective_state_update_ssu_amd import workloads as wl

    def med(call):
        return statistics.median(time_calls(call, steps, warmup)[1] * 1e3 for _ in range(3))

    for batch in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        w = wl.one_token("sweep", 1, batch=batch, H=80, P=64, N=128, G=1, nslots=2 * batch,
                         device="cuda", state_dtype="f32", io="bf16", with_z=True)
        acc = accounting(w)
        # Small batches cycle through copies of the state cache (at least 1 GiB of
        # state between two uses of one copy), and a graph holds one call per copy,
        # so neither figure is served from the Infinity Cache.
        copies = state_copies(acc)
        calls = rotated_calls(w, 0, copies=copies)
        eager = med(calls)
        prepared = med(prepared_calls(w, copies))
        length = max(steps, copies)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            calls[0]()  # warm the binding on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(length):
                calls[i % copies]()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / length)
        nbytes = acc["bytes"]
        replayed = statistics.median(ts)
        print(json.dumps({"sweep": "batch", "batch": batch, "state_copies": copies,
                          "eager_us": eager, "prepared_us": prepared, "graph_us": replayed,
                          "graph_gbps": nbytes / replayed / 1e3}), flush=True)
        del graph, w, calls
        torch.cuda.empty_cache()
    for sd, esz in (("f32", 4), ("bf16", 2)):
        for N in (16, 32, 64, 128, 256):
            batch = int(round(1.35e9 / (2 * 80 * 64 * N * esz)))
            w = wl.one_token("sweep_ds", 7, batch=batch, H=80, P=64, N=N, G=1,
                             nslots=2 * batch, device="cuda", state_dtype=sd, io="bf16",
                             with_z=True)
            acc = accounting(w)
            t = med(rotated_calls(w, 0, copies=state_copies(acc)))
            print(json.dumps({"sweep": "dstate", "state": sd, "dstate": N, "batch": batch,
                              "us": t, "gbps": acc["bytes"] / t / 1e3}), flush=True)
            del w
            torch.cuda.empty_cache()


def main():
    args = parse()
    if args.mode == "summarize":
        if args.workload.startswith("ssd_"):
            summarize_ssd(args.prof_dir, args.workload, args.prof_cmd)
        else:
            summarize(args.prof_dir, args.workload, args.prof_cmd)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              f"supported: the selective state update has no cross-GPU step to scale.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.mode == "copy":
        print(json.dumps({"ceilings_gbps": ceilings(steps=args.steps, kinds=("copy",)),
                          "bytes_each_way": 2 << 30}))
        return
    if args.mode == "sweep":
        sweep(min(args.steps, 100), args.warmup)
        return

    def record(rec):
        if args.record:
            with open(args.record, "w") as f:
                json.dump(rec, f)

    if args.mode == "kernel" and args.workload.startswith("ssd_"):
        rec = run_ssd_workload(args.workload, args.steps, args.warmup)
        print(f"[bench] {args.workload}: {rec['us_per_prefill']:.1f} us/prefill",
              file=sys.stderr, flush=True)
        record(rec)
        print(json.dumps(rec))
        return
    head = run_workload(args.workload, args.steps, args.warmup, args.heads_per_block,
                        args.loads_per_lane)
    print(f"[bench] {args.workload}: {head['kernel_us']:.1f} us/launch, "
          f"{head['hbm_gbps']:.0f} GB/s, {head['tokens_per_s'] / 1e6:.3f} M tokens/s",
          file=sys.stderr, flush=True)
    if args.mode == "kernel":
        record(head)
        print(json.dumps(head))
        return

    extra = {}
    if not args.no_extra:
        for name in ("mamba2_2p7b", "tiny", "bf16_state", "bf16_state_sr", "nemotron_h",
                     "nemotron_h_readonly", "packed_mtp", "dense_mtp"):
            if name == args.workload:
                continue
            rec = run_workload(name, max(20, args.steps // 2), max(5, args.warmup // 2),
                               args.heads_per_block, args.loads_per_lane)
            extra[name] = {k: rec[k] for k in ("tokens_per_s", "hbm_gbps", "frac_of_peak",
                                               "kernel_us", "ms_per_step", "bytes", "live_rows",
                                               "state_copies", "cache_resident", "roofline",
                                               "state_traffic_only_us",
                                               "frac_of_state_traffic_only") if k in rec}
            print(f"[bench] {name}: {rec['kernel_us']:.1f} us/launch, {rec['hbm_gbps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        for name in ("ssd_mamba2_2p7b", "ssd_nemotron_h"):
            rec = run_ssd_workload(name, max(10, args.steps // 10), max(3, args.warmup // 4))
            extra[name] = {k: rec[k] for k in ("config", "tokens_per_s", "us_per_prefill",
                                               "ms_per_step", "hbm_gbps", "frac_of_peak",
                                               "tflops", "bytes", "flops")}
            print(f"[bench] {name}: {rec['us_per_prefill']:.1f} us/prefill, "
                  f"{rec['tokens_per_s'] / 1e6:.2f} M tokens/s, {rec['hbm_gbps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        if not args.no_cpu_baseline:
            try:  # an extra figure: its failure is reported, not fatal to the line
                extra["ssd_cpu_baseline"] = ssd_cpu_baseline(min(5.0, args.cpu_seconds))
            except Exception as e:  # noqa: BLE001
                extra["ssd_cpu_baseline"] = {"error": f"{type(e).__name__}: {e}"}
    ceil = ceilings()
    copy_gbps = ceil["copy"]
    rings = ring_tracker_times()
    print(f"[bench] ring trackers: {json.dumps(rings)}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, args.workload)

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "hbm_gbps": head["hbm_gbps"],
        "frac_of_peak": head["frac_of_peak"],
        "copy_gbps": copy_gbps,
        "frac_of_copy": head["hbm_gbps"] / copy_gbps,
        "stream_ceilings_gbps": ceil,
        "state_copies": head["state_copies"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "workloads": extra,
        "ring_trackers": rings,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
