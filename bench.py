#!/usr/bin/env python3
"""Benchmark of the factorized sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
st_sparse_attn_fwd followed by st_sparse_attn_bwd (Delta preprocess, dq,
dk/dv and the split reduction), with the block LUTs and schedules already
cached (their one-off build time is reported separately).  The default
workload is the fixed pattern at T = 12288 with forward + recompute backward
(B=4, H=8, l=128, c=8, D=64, bf16), the configuration the headline metric
(useful fwd+bwd TFLOP/s and tokens/s at T=12288) is quoted on.

Output: one JSON line.  ``value`` is useful TFLOP/s: 14*D*nnz FLOP per step
(forward 4*D*nnz: QK^T and PV; backward 10*D*nnz: S recomputed, dP, dV, dQ,
dK) over the step time, nnz = sum over heads of |S(t)|; masked or skipped
work is never counted (``executed_tflops`` counts every pair of the visited
64x64 LUT blocks instead, and is labelled as such).  The step time is taken over ``--steps`` steps
between two HIP events on the launch stream, after a warm-up of at least
``--warmup`` steps and ``--warmup-seconds`` seconds.  ``ms_per_step_median``
adds the median single-step time back to back (warm) and after a 512 MiB
write that evicts the last-level cache (cold).  ``roofline`` describes the
kernel with the largest time per step: its duration comes from HIP events
that the library records around each kernel launch on the same stream, in a
second timed pass of the same ``--steps`` steps (those events add a few
microseconds between kernels, so that pass's step time is reported
separately and is not ``value``).  ``cpu_baseline`` times the fp64 oracle on
the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MI355X_HBM_GBS = 8000.0        # HBM3E peak, GB/s
MI355X_BF16_TFLOPS = 2500.0    # dense bf16 (and fp16) MFMA peak, TFLOP/s
MI355X_FP32_TFLOPS = 157.3     # dense fp32 MFMA peak, TFLOP/s


# ---------------------------------------------------------------------------
# Work accounting (closed forms per head kind)
# ---------------------------------------------------------------------------

def active_rows(pattern, kind, T, l, c):
    """Query rows whose key set (of this kind, or of this pass for merged heads) is non-empty."""
    from factorized_sparse_self_amd import ST_FIXED, ST_FIXED_R1, ST_FIXED_UNION, ST_STRIDED_UNION
    from factorized_sparse_self_amd.inputs import summary_offsets
    if pattern in (ST_FIXED, ST_FIXED_UNION, ST_STRIDED_UNION) and kind == 1:
        return max(0, T - l)
    if pattern == ST_FIXED_R1 and kind == 1:
        return max(0, T - summary_offsets(l, c)[0])
    return T


def attended_keys(pattern, kind, T, l, c):
    """Key positions some query attends (in this kind, or this pass for merged heads)."""
    from factorized_sparse_self_amd import ST_FIXED, ST_FIXED_R1, ST_FIXED_UNION, ST_STRIDED_UNION
    from factorized_sparse_self_amd.inputs import summary_offsets
    nb = -(-T // l)
    if pattern in (ST_FIXED, ST_FIXED_UNION) and kind == 1:
        return (nb - 1) * len(summary_offsets(l, c))
    if pattern == ST_FIXED_R1 and kind == 1:
        return sum(1 for b in range(nb) for s in summary_offsets(l, c) if b * l + s < T)
    if pattern == ST_STRIDED_UNION and kind == 1:
        return max(0, T - l)
    return T


def second_pass_keys(pattern, T, l, c):
    """Merged heads: key positions the second pass holds (their first-pass dk / dv are
    carried in fp32 and merged)."""
    from factorized_sparse_self_amd import ST_FIXED_UNION
    from factorized_sparse_self_amd.inputs import summary_offsets
    nb = -(-T // l)
    return (nb - 1) * len(summary_offsets(l, c)) if pattern == ST_FIXED_UNION else T


def head_passes(pattern, h):
    """(kind, store) of each pass over head h: one pass of the head's own kind, or for
    merged heads a carrying pass of kind 0 and a merging pass of kind 1."""
    from factorized_sparse_self_amd import ST_FIXED_UNION, ST_STRIDED_UNION
    if pattern in (ST_STRIDED_UNION, ST_FIXED_UNION):
        return [(0, "carry"), (1, "merge")]
    return [(h % 2, "final")]


def accounting(w):
    """Per-kernel algorithmic bytes and useful FLOP for one step of workload w."""
    from factorized_sparse_self_amd import st_layout_build
    lay = st_layout_build(w.pattern, w.T, w.l, w.c)
    E = 4 if w.dtype == "f32" else 2
    row = w.D * E
    crow = w.D * 4  # fp32 carried row of a merged head
    by = {"fwd": 0, "bwd_pre": 0, "bwd_dq": 0, "bwd_dkdv": 0, "bwd_reduce": 0}
    pairs_total = 0
    visited = 0
    for h in range(w.H):
        for kind, store in head_passes(w.pattern, h):
            pairs = lay[kind]["pairs"]
            rows = active_rows(w.pattern, kind, w.T, w.l, w.c)
            keys = attended_keys(w.pattern, kind, w.T, w.l, w.c)
            pairs_total += w.B * pairs
            visited += w.B * lay[kind]["nnz"]
            # forward: read q (active rows), k and v (attended keys); write out and lse
            # (every row), or the fp32 carried output and lse, or read those and write
            out_fwd = {"final": w.T * (row + 4), "carry": w.T * (crow + 4),
                       "merge": w.T * (crow + 4) + w.T * (row + 4)}[store]
            by["fwd"] += w.B * (rows * row + 2 * keys * row + out_fwd)
            # Delta and the zero fill: read out and dout, write Delta; zero dk and dv where no
            # query attends (a kernel of its own for fp32)
            pre = w.T * (2 * row + 4) + 2 * (w.T - keys) * row
            # dq: read q, dout, lse, Delta (active rows), k and v (keys); write dq (every row)
            dq = rows * (2 * row + 8) + 2 * keys * row + w.T * row
            if w.dtype != "f32":
                # the 16-bit dq computes Delta itself: reads q, dout, lse (active rows), out (every
                # row), k and v (keys); writes dq (or its carried fp32 row, or reads that and
                # writes dq), Delta and lse*log2(e) (every row, not in a merging pass) and
                # the zero fill (plain heads)
                out_dq = {"final": w.T * row, "carry": w.T * crow, "merge": w.T * (crow + row)}[store]
                side = 8 * w.T if store != "merge" else 0
                zero = 2 * (w.T - keys) * row if store == "final" else 0
                by["bwd_dq"] += w.B * (rows * (2 * row + 4) + 2 * keys * row + w.T * row + out_dq + side + zero)
            else:
                by["bwd_pre"] += w.B * pre
                by["bwd_dq"] += w.B * dq
            # dk/dv: read q, dout, lse, Delta (active rows), k and v (keys); write dk and dv
            # (keys); merged heads carry the keys the second pass holds in fp32
            if store == "final":
                out_kv = 2 * keys * row
            elif store == "carry":
                held = second_pass_keys(w.pattern, w.T, w.l, w.c)
                out_kv = 2 * (held * crow + (w.T - held) * row)
            else:
                out_kv = 2 * second_pass_keys(w.pattern, w.T, w.l, w.c) * (crow + row)
            by["bwd_dkdv"] += w.B * (rows * (2 * row + 8) + 2 * keys * row + out_kv)
    fl = {"fwd": 4 * w.D * pairs_total, "bwd_pre": 0, "bwd_dq": 6 * w.D * pairs_total,
          "bwd_dkdv": 8 * w.D * pairs_total, "bwd_reduce": 0}
    useful = (4 if not w.backward else 14) * w.D * pairs_total
    # executed: every pair of every visited 64x64 LUT block (masked ones included)
    executed = (4 if not w.backward else 14) * w.D * visited * lay[0]["block"] ** 2
    head_pairs = [sum(lay[kind]["pairs"] for kind, _ in head_passes(w.pattern, h)) for h in range(2)]
    return {"bytes": by, "flops": fl, "useful_flops": useful, "executed_flops": executed, "pairs": pairs_total,
            "head_pairs": head_pairs}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ---------------------------------------------------------------------------

# The oracle timing is bounded: when the whole workload would take the pool more
# than about ORACLE_BUDGET_S seconds, every slice is timed on an evenly spaced
# subset of its rows instead (and only those rows' FLOP are counted).
ORACLE_BUDGET_S = 20.0
# Worker processes: the host's cores, at most this many (the CPU share of one GPU on a shared node).
ORACLE_MAX_WORKERS = 16


def _one_thread():
    """Pool initializer: one BLAS / OpenMP thread per oracle process (set before
    numpy is imported in the worker), so that `cores` is the thread count."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"


def _oracle_unit(args):
    wname, b, h0, rows = args
    import torch
    import oracle
    from factorized_sparse_self_amd import inputs
    w = inputs.WORKLOAD_BY_NAME[wname]
    tensors = inputs.draw_workload(w)
    arrs = [x[b:b + 1, h0:h0 + 2].to(torch.float64).numpy() for x in tensors]
    t0 = time.perf_counter()
    if rows is not None:
        # row sample: the forward and the dq part of the backward at these rows
        oracle.forward_rows(arrs[0], arrs[1], arrs[2], w.pattern, w.l, w.c, rows)
        if w.backward:
            oracle.backward_dq_rows(arrs[0], arrs[1], arrs[2], arrs[3], w.pattern, w.l, w.c, rows)
    elif w.backward:
        oracle.backward(arrs[0], arrs[1], arrs[2], arrs[3], w.pattern, w.l, w.c)
    else:
        oracle.forward(arrs[0], arrs[1], arrs[2], w.pattern, w.l, w.c)
    return time.perf_counter() - t0


def cpu_baseline(w, acct):
    """Time the oracle on every (batch, head-pair) slice of the workload with a pool of
    one single-threaded process per host core (at most ORACLE_MAX_WORKERS).

    A slice is the full sequence of two heads (one of each kind), forward and (if the
    workload has one) backward.  value = the FLOP of the timed work over the pool's
    wall time.  When the whole workload would take more than about ORACLE_BUDGET_S
    seconds, each slice is timed on an evenly spaced subset of its rows (forward and
    the dq part of the backward at those rows) and only those rows' FLOP count.
    """
    import numpy as np
    import oracle
    flop_per_pair = (14 if w.backward else 4) * w.D
    slice_flops = sum(acct["head_pairs"]) * flop_per_pair
    workers = max(1, min(os.cpu_count() or 1, ORACLE_MAX_WORKERS))
    slices = [(b, h0) for b in range(w.B) for h0 in range(0, w.H - 1, 2)]
    rows = None
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(workers, len(slices)), initializer=_one_thread) as pool:
        n_pool = min(workers, len(slices))
        # pilot: 16 evenly spaced rows of the first n_pool slices at once (the
        # processes slow each other down), scaled to whole slices (the full backward
        # adds the dk/dv part: x 1.4) and to the pool's rounds over all slices
        pilot = np.unique(np.linspace(0, w.T - 1, 16).astype(np.int64))
        per_row = max(pool.map(_oracle_unit, [(w.name, b, h0, pilot) for b, h0 in slices[:n_pool]])) / len(pilot)
        rounds = -(-len(slices) // n_pool)
        estimate = per_row * w.T * (1.4 if w.backward else 1.0) * rounds
        print(f"cpu baseline: whole workload estimated at {estimate:.1f} s on {n_pool} processes",
              file=sys.stderr, flush=True)
        if estimate > ORACLE_BUDGET_S:
            n = max(16, int(ORACLE_BUDGET_S / 2 / per_row / rounds))
            rows = np.unique(np.linspace(0, w.T - 1, min(n, w.T)).astype(np.int64))
            row_pairs = sum(oracle.key_set(w.pattern, kind, int(t), w.T, w.l, w.c).size
                            for kind in (0, 1) for t in rows)
            slice_flops = row_pairs * (10 if w.backward else 4) * w.D
        jobs = [(w.name, b, h0, rows) for b, h0 in slices]
        print(f"cpu baseline: timing {len(jobs)} slices" + ("" if rows is None else f" on {len(rows)} rows"),
              file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        per_unit = pool.map(_oracle_unit, jobs)
        wall = time.perf_counter() - t0
    flops = len(jobs) * slice_flops
    what = ("full T={}, {}".format(w.T, "forward + backward" if w.backward else "forward") if rows is None else
            "{} evenly spaced rows of T={} per slice, forward{} at those rows (a row sample: the rate is "
            "extrapolated to the workload as FLOP per second)".format(
                len(rows), w.T, " + the dq part of the backward" if w.backward else ""))
    return {
        "value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": n_pool, "kind": "oracle",
        "sample": (f"all {len(jobs)} (batch, head-pair) slices of {w.name}: {what}; fp64 numpy, one "
                   f"single-threaded process per core ({n_pool} processes); value = timed useful FLOP / "
                   f"pool wall time"),
        "seconds_per_slice": [round(x, 3) for x in per_unit], "wall_s": round(wall, 3),
        "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
    }


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family / model / stepping."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    return (f"{name} (family {info.get('cpu family', '?')}, model {info.get('model', '?')}, "
            f"stepping {info.get('stepping', '?')})")


# ---------------------------------------------------------------------------
# HBM traffic from committed rocprofv3 counter summaries
# ---------------------------------------------------------------------------

def kernel_source_digest():
    h = hashlib.sha256()
    for name in ("st_fwd.hip", "st_bwd.hip", "st_device.hpp", "st_kernels.hpp", "st_geometry.hpp", "st_stage.hpp"):
        with open(os.path.join(ROOT, "factorized_sparse_self_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/, or None when absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_sha256") != kernel_source_digest():
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fixed_T12288_bf16_fwdbwd")
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="keep warming up (untimed) until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="evict the last-level cache before every step, warm-up and timed ones (for counter "
                         "runs of cold traffic; the JSON line's timings then include the eviction writes)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the sparse attention path runs and is timed on a single MI355X "
              "(heads are independent, so several GPUs would each run their own share of the heads); "
              "--gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from factorized_sparse_self_amd import (inputs, st_sparse_attn_bwd, st_sparse_attn_fwd,
                                            st_timing_enable, st_timing_read, st_timing_reset,
                                            KERNEL_NAMES, st_layout_build)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = inputs.WORKLOAD_BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    st_layout_build(w.pattern, w.T, w.l, w.c)
    layout_ms = (time.perf_counter() - t0) * 1e3
    acct = accounting(w)

    tensors = [x.to(dev) for x in inputs.draw_workload(w)]
    q, k, v = tensors[:3]
    do = tensors[3] if w.backward else None
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.T, dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flush_buf = torch.empty(512 << 18, dtype=torch.float32, device=dev)

    def evict(i):
        """Write 512 MiB, which leaves none of the inputs in the 256 MB last-level cache."""
        flush_buf.fill_(float(i))

    def step():
        if args.cold:
            evict(0)
        st_sparse_attn_fwd(q, k, v, w.pattern, w.l, w.c, out=out, lse=lse)
        if w.backward:
            st_sparse_attn_bwd(q, k, v, out, lse, do, w.pattern, w.l, w.c, dq=dq, dk=dk, dv=dv)

    # Warm-up: at least W steps and at least --warmup-seconds of them, so that
    # the GPU's clocks reach their steady state before the timed steps (after
    # the ~2 ms of ten steps alone, a step measures about 10% slower than it
    # does in a running loop).
    t_warm = time.perf_counter()
    warm_steps = 0
    while warm_steps < args.warmup or time.perf_counter() - t_warm < args.warmup_seconds:
        for _ in range(10):
            step()
        warm_steps += 10
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_warm

    stream = torch.cuda.current_stream(dev)

    def timed_steps(instrumented):
        """Time `steps` steps between two events on the launch stream; with
        `instrumented`, the library also brackets each kernel with HIP events."""
        st_timing_reset()
        st_timing_enable(instrumented)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        st_timing_enable(False)
        return start.elapsed_time(end) / args.steps

    def per_step_median(flush, instrumented=False):
        """Median of `steps` single-step times (an event pair around each step).
        With `flush`, a 512 MiB buffer is written before every step, outside
        the events, so that no input is left in the 256 MB last-level cache
        (cold); without it the steps run back to back (warm).  With
        `instrumented`, the library also times each kernel (read afterwards)."""
        marks = []
        st_timing_reset()
        st_timing_enable(instrumented)
        torch.cuda.synchronize()
        for i in range(args.steps):
            if flush:
                evict(i)
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record(stream)
            step()
            e_.record(stream)
            marks.append((s_, e_))
        torch.cuda.synchronize()
        st_timing_enable(False)
        return statistics.median(s_.elapsed_time(e_) for s_, e_ in marks)

    def kernel_times():
        out = {}
        for name in KERNEL_NAMES:
            n, tot = st_timing_read(name)
            if n:
                out[name] = {"launches_per_step": n / args.steps, "avg_ms": tot / n,
                             "ms_per_step": tot / args.steps}
        return out

    # The step time comes from a pass without per-kernel events (each event
    # pair adds a few microseconds between kernels); the per-kernel durations
    # for the roofline come from an identical pass with them.  The same for
    # single steps after a last-level-cache eviction (cold).
    ms_per_step = timed_steps(False)
    ms_per_step_instrumented = timed_steps(True)
    kernels = kernel_times()
    median_warm = per_step_median(False)
    median_cold = per_step_median(True)
    per_step_median(True, instrumented=True)
    kernels_cold = kernel_times()

    useful_tflops = acct["useful_flops"] / (ms_per_step * 1e-3) / 1e12
    executed_tflops = acct["executed_flops"] / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = w.B * w.T / (ms_per_step * 1e-3)
    dom = max(kernels, key=lambda k_: kernels[k_]["ms_per_step"])
    # per launch: a step's bytes and FLOP of the kernel over its launches per step
    # (merged heads launch each kernel once per pass)
    dur_s = kernels[dom]["avg_ms"] * 1e-3
    dom_bytes = acct["bytes"][dom] / kernels[dom]["launches_per_step"]
    dom_flops = acct["flops"][dom] / kernels[dom]["launches_per_step"]
    peak_flops = MI355X_FP32_TFLOPS if w.dtype == "f32" else MI355X_BF16_TFLOPS
    ridge = peak_flops * 1e12 / (MI355X_HBM_GBS * 1e9)
    ai = dom_flops / dom_bytes if dom_bytes else float("inf")
    if ai < ridge:
        achieved, peak, unit, bound = dom_bytes / dur_s / 1e9, MI355X_HBM_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = dom_flops / dur_s / 1e12, peak_flops, "TFLOP/s", "mfma"
    roofline = {
        "kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
        "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, w.name),
        "algorithmic_bytes": dom_bytes, "useful_flops": dom_flops, "avg_ms": round(kernels[dom]["avg_ms"], 4),
        "useful_tflops": round(dom_flops / dur_s / 1e12, 2),
        "mfma_frac": round(dom_flops / dur_s / 1e12 / peak_flops, 4),
    }
    # the same kernel with its inputs evicted from the last-level cache before every step
    roofline_cold = None
    if dom in kernels_cold:
        dur_c = kernels_cold[dom]["avg_ms"] * 1e-3
        ach_c = (dom_bytes / dur_c / 1e9) if bound == "hbm" else (dom_flops / dur_c / 1e12)
        roofline_cold = {"kernel": dom, "bound": bound, "achieved": round(ach_c, 2), "peak": peak, "unit": unit,
                         "frac": round(ach_c / peak, 4), "traffic": measured_traffic(dom, w.name + "_cold"),
                         "avg_ms": round(kernels_cold[dom]["avg_ms"], 4)}

    result = {
        "metric": "sparse-attn fwd+bwd useful TFLOP/s & tokens/s at T=12288, % of bf16 MFMA peak",
        "value": round(useful_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_with_kernel_events": round(ms_per_step_instrumented, 4),
        "ms_per_step_median": {"warm": round(median_warm, 4), "cold": round(median_cold, 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pattern": inputs.PATTERN_NAMES[w.pattern], "B": w.B, "H": w.H,
                   "T": w.T, "D": w.D, "l": w.l, "c": w.c, "passes": "fwd+bwd" if w.backward else "fwd",
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU"},
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_bf16_mfma_peak": round(100 * useful_tflops / MI355X_BF16_TFLOPS, 3),
        "useful_gflop_per_step": round(acct["useful_flops"] / 1e9, 3),
        "executed_tflops": round(executed_tflops, 3),
        "executed_gflop_per_step": round(acct["executed_flops"] / 1e9, 3),
        "nnz_pairs": acct["pairs"],
        "kernels": {k_: {kk: round(vv, 5) for kk, vv in v_.items()} for k_, v_ in kernels.items()},
        "kernels_cold": {k_: round(v_["avg_ms"], 5) for k_, v_ in kernels_cold.items()},
        "layout_build_ms": round(layout_ms, 3),
        "roofline": roofline,
        "roofline_cold": roofline_cold,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, acct)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
