#!/usr/bin/env python3
"""Benchmark of the fused relative-position attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the fused forward (every kernel of the path: the
row-constant pre-pass of Transformer-XL, the fused attention kernel, the
split-KV merge) over one batch of seeded synthetic inputs already
resident in HBM.  Every figure is the median over timed replays of a HIP
graph of exactly `--steps` steps (at least 5 replays and 200 ms), with the
fastest and slowest replay beside it.  Prints one JSON line: the headline is
DeBERTa k=512, with Shaw k=16 causal (the other workload the metric is
quoted on) under "targets" and the remaining workloads under "secondary".

Counted FLOPs follow the FlashAttention convention: 4*d per visible
(query, key) pair (q.k and p.v), plus for Shaw 2*d per distinct (row,
clipped offset) for q.a_K and again for the binned a_V product, plus for
DeBERTa 2*d per distinct (row, delta) for content-to-position and 2*d per
distinct (key, delta) for position-to-content.  Masked pairs, the bias add
and the softmax are not counted.  Algorithmic bytes: Q and O once, the K/V
rows any query can see once, the relative tables once.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from transformer_attention_relative_amd.synthetic import WORKLOADS, Workload, make_inputs, params_of  # noqa: E402

# The metric is quoted on the two bf16 workloads of length >= 2048 that are
# bound by the matrix cores: DeBERTa k=512 (the largest counted work, the
# headline `value`) and Shaw k=16 causal, both timed the same way.
DEFAULT_WORKLOAD = "deberta_k512"
TARGETS = ["deberta_k512", "shaw_causal_k16"]
SECONDARY = ["t5_encoder_padded", "t5_decoder_kvcache", "t5_decode_evicted", "alibi_causal",
             "alibi_causal_d128", "txl_memory"]
METRIC = "rel-pos attention fwd TFLOP/s and % of MFMA bf16 peak (1 MI355X)"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X published dense MFMA peaks
PEAK_HBM_GBS = 8000.0                             # MI355X published HBM3E bandwidth
KERNEL_SOURCES = ["transformer_attention_relative_amd/csrc/relattn_kernels.hip",
                  "transformer_attention_relative_amd/csrc/relattn_api.cpp",
                  "transformer_attention_relative_amd/csrc/relattn_internal.hpp"]


# ----------------------------------------------------------------------------
# counted work
# ----------------------------------------------------------------------------

def _kv_limits(wl: Workload, kv_valid_len):
    if kv_valid_len is None:
        return np.full(wl.B, wl.Lk, dtype=np.int64)
    return np.minimum(np.asarray(kv_valid_len, dtype=np.int64), wl.Lk)


def counted_work(wl: Workload, kv_valid_len):
    """(counted FLOPs, algorithmic bytes) of one forward call."""
    lims = _kv_limits(wl, kv_valid_len)
    # query positions counted from key row 0 (every term depends on the
    # difference of the absolute positions only)
    qoff = wl.q_pos_offset - wl.k_pos_offset
    pos = qoff + np.arange(wl.Lq, dtype=np.int64)
    esz = 4 if wl.dtype == "fp32" else 2
    flops = 0.0
    kv_bytes = 0.0
    k = wl.clip_k
    for b in range(wl.B):
        lim = int(lims[b])
        nvis = np.minimum(lim, pos + 1) if wl.causal else np.full(wl.Lq, lim)
        nvis = np.maximum(nvis, 0)
        per_head = 4.0 * wl.d * nvis.sum()
        if wl.kind == "shaw":
            has = nvis > 0
            lo = np.clip(-pos, -k, k)
            hi = np.clip(nvis - 1 - pos, -k, k)
            per_head += 4.0 * wl.d * np.where(has, hi - lo + 1, 0).sum()
        elif wl.kind == "txl":
            # (q + v).E[i - j]: one distinct (row, distance) per visible pair
            per_head += 2.0 * wl.d * nvis.sum()
        elif wl.kind == "deberta":
            has = nvis > 0
            hi = np.clip(pos, -k, k - 1)
            lo = np.clip(pos - (nvis - 1), -k, k - 1)
            per_head += 2.0 * wl.d * np.where(has, hi - lo + 1, 0).sum()
            # per key column: the query rows that see key j
            j = np.arange(wl.Lk, dtype=np.int64)
            if wl.causal:
                first = np.maximum(j - qoff, 0)                     # first row with pos >= j
                nrows = np.where(j < lim, np.maximum(wl.Lq - first, 0), 0)
            else:
                first = np.zeros_like(j)
                nrows = np.where(j < lim, wl.Lq, 0)
            hasc = nrows > 0
            p_first = qoff + first
            p_last = qoff + wl.Lq - 1
            a_ = np.clip(j - p_last, -k, k - 1)
            b_ = np.clip(j - p_first, -k, k - 1)
            per_head += 2.0 * wl.d * np.where(hasc, b_ - a_ + 1, 0).sum()
        flops += wl.H * per_head
        reach = min(lim, int(pos[-1]) + 1) if wl.causal else lim
        kv_bytes += 2.0 * wl.H * max(reach, 0) * wl.d * esz
    qo_bytes = 2.0 * wl.B * wl.H * wl.Lq * wl.d * esz
    if wl.kind == "t5":
        tab = wl.num_buckets * wl.H * 4
    elif wl.kind == "shaw":
        tab = 2 * (2 * k + 1) * wl.d * esz
    elif wl.kind == "alibi":
        tab = wl.H * 4
    elif wl.kind == "txl":
        tab = (k + 2) * wl.H * wl.d * esz
    else:
        tab = 2 * (2 * k) * wl.H * wl.d * esz
    return flops, qo_bytes + kv_bytes + tab


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# GPU timing
# ----------------------------------------------------------------------------

def _prepare(wl: Workload, seed: int = 0):
    import torch
    import transformer_attention_relative_amd as ra
    inp = make_inputs(wl, seed)
    dev = {k: (None if v is None else v.to("cuda:0")) for k, v in inp.items()}
    out = torch.empty_like(dev["q"])
    p = ra.make_params(wl.kind, wl.dtype, wl.B, wl.H, wl.Lq, wl.Lk, wl.d, table=dev["table"],
                       table2=dev["table2"], kv_valid_len=dev["kv_valid_len"], **params_of(wl))
    nbytes = ra.relattn_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0")

    def step():
        ra.relattn_fwd(dev["q"], dev["k"], dev["v"], wl.kind, dev["table"], dev["table2"],
                       kv_valid_len=dev["kv_valid_len"], out=out, workspace=ws, **params_of(wl))
    return inp, dev, out, step


def time_steps(step, steps: int, warmup: int, use_graph: bool, min_replays: int = 5,
               min_total_ms: float = 200.0):
    """Per-step times (ms) of repeated timed runs of exactly `steps` steps:
    the steps are captured once in a HIP graph, which is replayed at least
    `min_replays` times and until `min_total_ms` of GPU time is covered;
    each replay is bracketed by synchronisations and timed with HIP events on
    the stream the kernels are launched on.  Returns (list of ms per step,
    one per replay, host wall ms per step of the first replay, graphed)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(steps):
                    step()
            graph.replay()          # untimed replay
            torch.cuda.synchronize()
        except Exception as e:      # launch mode only; the kernels are the same
            print(f"[bench] graph capture unavailable ({e}); timing eager launches",
                  file=sys.stderr)
            graph = None
    stream = torch.cuda.current_stream()
    per_step, walls, total = [], [], 0.0
    while len(per_step) < min_replays or total < min_total_ms:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for _ in range(steps):
                step()
        t1.record(stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - wall0) * 1e3 / steps)
        ms = t0.elapsed_time(t1)
        total += ms
        per_step.append(ms / steps)
        if len(per_step) >= 1000:
            break
    return per_step, walls[0], graph is not None


def time_cold(step, reps: int = 20, flush_bytes: int = 512 << 20):
    """Median ms of single steps, each after a 512 MiB write that evicts the
    inputs from L2 and the 256 MiB MALL (they stay resident in HBM).  The
    step and its events are queued behind the flush, so the events time the
    step alone."""
    import torch
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        buf.fill_(1.0)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        step()
        t1.record(stream)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    del buf
    return float(np.median(times))


COLD = ["t5_encoder_padded", "t5_decoder_kvcache"]   # the HBM-bound workloads


def roofline(wl: Workload, flops: float, nbytes: float, ms: float, traffic):
    peak_t = PEAK_TFLOPS[wl.dtype]
    t_mfma = flops / (peak_t * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    sec = ms * 1e-3
    if t_hbm > t_mfma:
        ach = nbytes / sec / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
    ach = flops / sec / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_t, "unit": "TFLOP/s",
            "frac": round(ach / peak_t, 4), "traffic": traffic}


# ----------------------------------------------------------------------------
# CPU baseline (the float64 oracle, as it stands)
# ----------------------------------------------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl: Workload, inp, budget_s: float = 15.0):
    import oracle
    affinity = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        blas = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max(blas) if blas else 1
    except Exception:
        blas_threads = 1
    # the oracle's matrix products run on the BLAS threads; the rest of it on
    # one thread; no more threads than the cores this process may use
    cores = max(1, min(blas_threads, affinity))
    f64 = lambda t: None if t is None else t.float().numpy().astype(np.float64)
    q, k, v = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    t1, t2 = f64(inp["table"]), f64(inp["table2"])
    lens = None if inp["kv_valid_len"] is None else inp["kv_valid_len"].numpy()
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    done = []
    t0 = time.perf_counter()
    # cycle over the (batch, head) slices until the time budget is spent
    # (at most 20 passes), so small workloads still give a stable rate
    while time.perf_counter() - t0 < budget_s and len(done) < 20 * len(heads):
        bh = heads[len(done) % len(heads)]
        oracle.relattn_forward(q, k, v, wl.kind, t1, t2, kv_valid_len=lens, heads=[bh],
                               **params_of(wl))
        done.append(bh)
    elapsed = time.perf_counter() - t0
    # counted FLOPs of the heads processed
    total = 0.0
    for b in sorted(set(b for b, _ in done)):
        nh = sum(1 for bb, _ in done if bb == b)
        sub = wl.replace(B=1, H=1)
        f, _ = counted_work(sub, None if lens is None else lens[b:b + 1])
        total += f * nh
    return {"value": round(total / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "workload": wl.name,
            "cpu_model": _cpu_model(), "sched_affinity_cores": affinity,
            "blas_threads": int(blas_threads),
            "sample": f"{len(done)} (batch, head) slices ({len(done) / len(heads):.2f} passes "
                      f"over the {len(heads)} of the workload), all query rows, float64 NumPy "
                      f"oracle, {elapsed:.1f} s"}


# ----------------------------------------------------------------------------

MIN_TIME_MS = 200.0


def measure(name: str, steps: int, warmup: int, use_graph: bool, cold: bool = False):
    """Time one workload; returns its record (median of the replays and
    their spread) and its seeded inputs."""
    wl = WORKLOADS[name]
    inp, dev, out, step = _prepare(wl)
    per_step, wall_ms, graphed = time_steps(step, steps, warmup, use_graph,
                                            min_total_ms=MIN_TIME_MS)
    flops, nbytes = counted_work(wl, inp["kv_valid_len"])
    ms = float(np.median(per_step))
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {"tflops": round(tflops, 2), "ms_per_step": round(ms, 5),
           "ms_per_step_min": round(min(per_step), 5), "ms_per_step_max": round(max(per_step), 5),
           "replays": len(per_step), "steps_per_replay": steps,
           "launch": "hip graph" if graphed else "eager",
           "counted_gflop": round(flops / 1e9, 3), "algorithmic_mb": round(nbytes / 1e6, 2),
           "mfma_peak_frac": round(tflops / PEAK_TFLOPS[wl.dtype], 4),
           "host_wall_ms_per_step": round(wall_ms, 5),
           "roofline": roofline(wl, flops, nbytes, ms, read_traffic(wl.name))}
    if cold:
        # single eager steps after an L2 / MALL flush (inputs in HBM only)
        cold_ms = time_cold(step)
        rec["cold_ms_per_step"] = round(cold_ms, 5)
        rec["cold_hbm_gbs"] = round(nbytes / (cold_ms * 1e-3) / 1e9, 1)
    return wl, inp, rec


def calibrate_copy(nbytes: int, reps: int):
    """Plain device-to-device copy of a known size, for scaling the HBM
    counters of rocprofv3 (FETCH_SIZE / WRITE_SIZE) to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def measured_mfma_peak():
    """Sustained v_mfma_f32_32x32x16_bf16 rate (TFLOP/s) from the probe library
    built beside librelattn.so, or None if it is not there."""
    import ctypes
    path = os.path.join(ROOT, "transformer_attention_relative_amd", "libmfma_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mfma_peak_bf16_tflops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mfma_peak_bf16_tflops.restype = ctypes.c_double
    best = max(lib.mfma_peak_bf16_tflops(512, 20000) for _ in range(3))
    return round(best, 1) if best > 0 else None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--min-time-ms", type=float, default=200.0,
                    help="replay the timed steps until this much GPU time is covered "
                         "(at least 5 replays; short profiler runs lower it)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other bf16 workloads in the JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by (batch, head) with no exchange, so N GPUs would each run "
              "this same single-GPU step on their share", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    global MIN_TIME_MS
    MIN_TIME_MS = args.min_time_ms
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(args.steps, 1))
        return

    probe = measured_mfma_peak()
    wl, inp, head = measure(args.workload, args.steps, args.warmup, not args.no_graph,
                            cold=args.workload in COLD)
    targets = {}
    for name in TARGETS:
        if name == wl.name:
            targets[name] = head
        elif not args.no_secondary:
            targets[name] = measure(name, args.steps, args.warmup, not args.no_graph,
                                    cold=name in COLD)[2]
    rec = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "kind": wl.kind,
                   "B": wl.B, "H": wl.H, "Lq": wl.Lq, "Lk": wl.Lk, "d": wl.d,
                   "parallelism": "none (1 GPU)",
                   "timing": "median over timed replays of a HIP graph of `steps` steps",
                   **{k: v for k, v in head.items() if k not in ("tflops", "ms_per_step", "roofline")}},
        "roofline": head["roofline"],
    }
    if probe and wl.dtype == "bf16":
        rec["config"]["mfma_measured_peak_tflops"] = probe
        rec["config"]["mfma_measured_peak_frac"] = round(head["tflops"] / probe, 4)
    if len(targets) > 1:
        # the metric's workloads side by side (same steps, warmup and timing)
        rec["targets"] = targets
    if not args.no_secondary:
        sec = {}
        for name in SECONDARY:
            if name == wl.name:
                continue
            w2, _, r2 = measure(name, args.steps, min(args.warmup, 5), not args.no_graph,
                                cold=name in COLD)
            sec[name] = r2
        rec["secondary"] = sec
    if probe:
        for r in list(rec.get("targets", {}).values()) + list(rec.get("secondary", {}).values()):
            r["mfma_measured_peak_frac"] = round(r["tflops"] / probe, 4)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
