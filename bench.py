#!/usr/bin/env python3
"""SSU decode throughput on one MI355X: tokens/s and achieved HBM GB/s.

A step is one call of the update over one synthetic decode batch with every
input already resident in HBM. The headline workload is the Mamba2-2.7B-shaped
one-token batch (256 sequences, 80 heads x 64 x 128, fp32 state in 512 slots,
bf16 x/B/C/z). The other named workloads are timed too and reported under
"workloads". The roofline figure divides the algorithmic bytes of one launch by
the launch's average duration from HIP events on the launch stream.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode full|kernel|copy]

--mode kernel times only the chosen workload (for profiler runs); --mode copy
times only the reference copy kernel used to calibrate traffic counters.
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
HEADLINE = "mamba2_2p7b"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--mode", choices=["full", "kernel", "copy"], default="full")
    ap.add_argument("--heads-per-block", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "selective_state_update_ssu_amd", "csrc", "*")))
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
    total = state_read + state_write + live_rows * row_bytes + index_bytes + 3 * 4 * H
    return dict(live_rows=live_rows, live_seqs=live_seqs, state_writes=writes,
                state_read_bytes=state_read, state_write_bytes=state_write, bytes=total)


# ---------------------------------------------------------------------- timing

def make_call(w, hpb):
    import torch
    import selective_state_update_ssu_amd as ssu

    state = w.state
    out = torch.empty_like(w.x)
    common = dict(D=w.D, z=w.z, dt_bias=w.dt_bias, dt_softplus=w.dt_softplus,
                  pad_slot_id=w.pad_slot_id, disable_state_update=w.disable_state_update,
                  heads_per_block=hpb)
    if w.mode == "one_token":
        return lambda: ssu.ssu_one_token(state, w.x, w.dt, w.A, w.B, w.C, out,
                                         state_batch_indices=w.src,
                                         dst_state_batch_indices=w.dst, **common)
    return lambda: ssu.ssu_packed_varlen(state, w.x, w.dt, w.A, w.B, w.C, w.cu_seqlens, out,
                                         num_accepted_tokens=w.num_accepted,
                                         state_batch_indices=w.src_table,
                                         dst_state_batch_indices=w.dst_table, **common)


def time_calls(call, steps, warmup):
    """Warm up, then time exactly `steps` calls. Returns (wall ms per step,
    event ms per launch on the launch stream)."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, start.elapsed_time(end) / steps


def copy_bandwidth(steps=50, nbytes=2 << 30):
    """A plain device copy of `nbytes` (torch's copy kernel): GB/s counting the
    bytes read plus the bytes written."""
    import torch

    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    wall, ev = time_calls(lambda: b.copy_(a), steps, 5)
    return 2 * nbytes / (ev * 1e-3) / 1e9, ev


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


# ------------------------------------------------------------------ CPU leg

def cpu_baseline(seconds):
    """The fp64 oracle, single-threaded, on the first 16 sequences of the
    headline workload (their rows and slots), repeated for about `seconds`."""
    import numpy as np
    import oracle
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.mamba2_2p7b("cpu")
    nseq = 16
    src = w.src[:nseq].long().numpy()
    used = sorted(set(src.tolist()))
    remap = {s: i for i, s in enumerate(used)}
    sub = dict(
        state=w.state[torch_index(used)].double().numpy(),
        x=w.x[:nseq].double().numpy(), dt=w.dt[:nseq].double().numpy(),
        A=w.A.double().numpy(), B=w.B[:nseq].double().numpy(), C=w.C[:nseq].double().numpy(),
        D=w.D.double().numpy(), z=w.z[:nseq].double().numpy(),
        dt_bias=w.dt_bias.double().numpy())
    s = np.array([remap[v] for v in src])
    orc = oracle.default()
    calls = 0
    t0 = time.perf_counter()
    while True:
        orc.one_token(sub["state"], sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"],
                      D=sub["D"], z=sub["z"], dt_bias=sub["dt_bias"], dt_softplus=True,
                      src=s, dst=s)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": nseq * calls / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nseq} of 256 sequences of {HEADLINE} (all 80 heads, their "
                      f"16 slots), fp64, {calls} calls in {el:.1f} s, one thread"}


def torch_index(idx):
    import torch
    return torch.as_tensor(idx, dtype=torch.long)


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


def run_workload(name, steps, warmup, hpb):
    import torch
    from selective_state_update_ssu_amd import workloads as wl

    w = wl.NAMED[name]("cuda")
    acc = accounting(w)
    wall, ev = time_calls(make_call(w, hpb), steps, warmup)
    rec = dict(config=describe(w), ms_per_step=wall, kernel_us=ev * 1e3,
               tokens_per_s=acc["live_rows"] / (wall * 1e-3),
               hbm_gbps=acc["bytes"] / (ev * 1e-3) / 1e9, **acc)
    rec["frac_of_peak"] = rec["hbm_gbps"] / HBM_PEAK_GBPS
    del w
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
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
        gbps, ms = copy_bandwidth()
        print(json.dumps({"copy_gbps": gbps, "copy_ms": ms, "bytes_each_way": 2 << 30}))
        return

    head = run_workload(args.workload, args.steps, args.warmup, args.heads_per_block)
    print(f"[bench] {args.workload}: {head['kernel_us']:.1f} us/launch, "
          f"{head['hbm_gbps']:.0f} GB/s, {head['tokens_per_s'] / 1e6:.3f} M tokens/s",
          file=sys.stderr, flush=True)
    if args.mode == "kernel":
        print(json.dumps(head))
        return

    extra = {}
    if not args.no_extra:
        for name in ("tiny", "bf16_state", "nemotron_h", "nemotron_h_readonly", "packed_mtp"):
            if name == args.workload:
                continue
            rec = run_workload(name, max(20, args.steps // 2), max(5, args.warmup // 2),
                               args.heads_per_block)
            extra[name] = {k: rec[k] for k in ("tokens_per_s", "hbm_gbps", "frac_of_peak",
                                               "kernel_us", "ms_per_step", "bytes", "live_rows")}
            print(f"[bench] {name}: {rec['kernel_us']:.1f} us/launch, {rec['hbm_gbps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
    copy_gbps, _ = copy_bandwidth()
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    kernel_ms = head["kernel_us"] * 1e-3
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
        "roofline": {
            "bound": "hbm",
            "achieved": head["hbm_gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": head["frac_of_peak"],
            "traffic": traffic_for(args.workload, kernel_ms),
            "algorithmic_bytes": head["bytes"],
            "kernel_us": head["kernel_us"],
        },
        "cpu_baseline": cpu,
        "workloads": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
