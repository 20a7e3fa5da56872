#!/usr/bin/env python3
"""Benchmark of the QSA sparse-attention decode step on one MI355X.

Workload (default): 8 sequences x 262,144 cached tokens, 12 QSA layers,
indexer_budget 2048 (512 C4 blocks), first block forced as a sink, 32 planted
relevant blocks per sequence per layer; index keys (66 B/token/layer) and the
bf16 KV pools (2048 B/token/layer, 51.5 GB) are resident in HBM before timing.
A step is one full pass of the hot path over all 12 layers (score -> select ->
paged attention -> merge) through the C ABI; the metric is layer-steps/s.

Prints one JSON line with the driver's fields plus:
  roofline      the dominant kernel (index scoring) as the headline step
                launches it: algorithmic bytes per launch / its average
                duration, timed with HIP events taken by the launch itself.
                Without a hot cache one launch scans all the layers (up to
                16), so a launch's bytes are the layers' index bytes together;
  one_stream_score  the same for the scoring launch of a one-layer call
                (each launch has the GPU alone);
  one_stream    the step time with no side stream (the same grouped launches
                on one stream for HBM pools; groups of scan, selection,
                gather and attention for pinned-host pools; layer by layer
                with a hot cache);
  per_layer_calls  one qsa_decode_step call per layer, as a model with
                dependent layers runs it;
  step_hbm      the whole step's algorithmic bytes (index scan + gathered
                rows) over the step time, against the same HBM peak;
  cpu_baseline  the CPU oracle, single-threaded, on a sample of (layer,
                sequence) units of the same workload, scaled to layer-steps/s;
  cold_cache    (HBM pools) steps timed one by one, each after reading a
                separate 512 MiB buffer, against the back-to-back steps: what
                the steps gain from data left in the 256 MB Infinity Cache.

The roofline's "traffic" comes from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
summarised in profiles/ (see --pmc-summary); it is reported only while the
scoring kernel's source is the one those counters were taken on.

Helper modes for the profiles (no benchmark run):
  --copy-calibration      a plain 256 MiB device-to-device copy, three times:
                          the known-size kernel that calibrates the counters;
  --stats-summary CSV     a short table of a rocprofv3 kernel_stats.csv;
  --pmc-summary F W CF CW summarise four rocprofv3 counter_collection.csv
                          files (bench FETCH_SIZE, bench WRITE_SIZE, copy
                          FETCH_SIZE, copy WRITE_SIZE) into the text file that
                          this script reads back.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
STEP_TARGET_FRAC = 0.70       # the whole step's index-scan + gather traffic, as a fraction of HBM peak
DRIFT = 0.25                  # indexer-query noise of the drifting region
COLD_FLUSH_BYTES = 512 << 20  # read before each step of the cold-cache region (Infinity Cache: 256 MB)
DRIFT_VARIANTS = 8
PCIE_PEAK_GBS = 64.0          # PCIe 5.0 x16, one direction
SCORE_KERNEL = "index_score_kernel"
SCORE_SOURCES = ("kv_cache_selection_amd/csrc/index_score.hip", "kv_cache_selection_amd/csrc/qsa_internal.h")
ATTN_KERNEL = "attn_split_kernel"
ATTN_SOURCES = ("kv_cache_selection_amd/csrc/attention.hip", "kv_cache_selection_amd/csrc/qsa_internal.h")
COPY_BYTES = 1 << 28


def pmc_file(workload):
    return os.path.join(ROOT, "profiles", "%s.%s.pmc.txt" % (SCORE_KERNEL, workload))


def score_source_hash(sources=SCORE_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_counter_csv(path):
    """{kernel name: [counter values]} from a rocprofv3 counter_collection.csv
    (one row per dispatch and counter)."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            low = {k.lower(): v for k, v in row.items()}
            name = low.get("kernel_name") or low.get("kernel-name") or ""
            out.setdefault(name, []).append(float(low["counter_value"]))
    return out


def pmc_summary(paths, workload):
    """Text summary of the four counter passes: KiB per dispatch for every
    kernel, the copy calibration factors and the scoring kernel's HBM bytes."""
    fetch, write, cfetch, cwrite = (read_counter_csv(p) for p in paths)

    def biggest(d):
        # the calibration copy is the only large dispatch of its run
        return max(v for vals in d.values() for v in vals)

    f_fetch = COPY_BYTES / (biggest(cfetch) * 1024.0)
    f_write = COPY_BYTES / (biggest(cwrite) * 1024.0)
    lines = ["# HBM traffic per dispatch from rocprofv3 counters, workload %s" % workload,
             "# four passes, each its own run (cd /tmp && export TMPDIR=/tmp first), C in FETCH_SIZE WRITE_SIZE:",
             "#   rocprofv3 --pmc C --kernel-trace -f csv -d OUT_C -o run -- python3 bench.py --steps 2 --warmup 1 "
             "--cpu-seconds 0 --no-sweep",
             "#   rocprofv3 --pmc C --kernel-trace -f csv -d COPY_C -o run -- python3 bench.py --copy-calibration",
             "# summary: python3 bench.py --pmc-summary OUT_FETCH_SIZE/run_counter_collection.csv "
             "OUT_WRITE_SIZE/run_counter_collection.csv COPY_FETCH_SIZE/run_counter_collection.csv "
             "COPY_WRITE_SIZE/run_counter_collection.csv",
             "# the copy moves %d bytes each way: its FETCH_SIZE and WRITE_SIZE readings give the KiB-to-byte "
             "factors" % COPY_BYTES,
             "kernel: %s" % SCORE_KERNEL,
             "source_sha256: %s" % score_source_hash(),
             "attn_source_sha256: %s" % score_source_hash(ATTN_SOURCES),
             "fetch_factor: %.4f" % f_fetch,
             "write_factor: %.4f" % f_write]
    # the scoring kernel comes as a launch over a group of layers (the
    # overlapped step) and as a launch per layer (the one-stream step)
    score = {}
    attn = {}
    rows = []
    for name in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(name, []), write.get(name, [])
        fk = sum(fv) / len(fv) if fv else 0.0
        wk = sum(wv) / len(wv) if wv else 0.0
        byt = fk * 1024.0 * f_fetch + wk * 1024.0 * f_write
        rows.append((byt, name, len(fv), fk, wk))
        if SCORE_KERNEL in name:
            score["layer" if "ScoreLayersT<1>" in name else "group"] = byt
        if ATTN_KERNEL in name and "AttnLayersT<1>" not in name:
            attn["group"] = byt
    if not score:
        raise SystemExit("no %s dispatch in the counter files" % SCORE_KERNEL)
    if "group" in score:
        lines.append("traffic_bytes_per_group_launch: %d" % round(score["group"]))
    if "layer" in score:
        lines.append("traffic_bytes_per_layer_launch: %d" % round(score["layer"]))
    if "group" in attn:
        lines.append("attn_traffic_bytes_per_group_launch: %d" % round(attn["group"]))
    lines.append("")
    lines.append("%14s %8s %14s %14s  %s" % ("bytes/dispatch", "dispatch", "FETCH KiB", "WRITE KiB", "kernel"))
    for byt, name, n, fk, wk in sorted(rows, reverse=True):
        lines.append("%14d %8d %14.1f %14.1f  %s" % (byt, n, fk, wk, name[:110]))
    return "\n".join(lines) + "\n"


def stats_summary(path, workload, op="step", bench_args=""):
    """Short text table of a rocprofv3 --stats kernel_stats.csv."""
    import csv
    lines = ["# rocprofv3 kernel statistics of a benchmark run, workload %s" % workload,
             "# command (cd /tmp && export TMPDIR=/tmp first):",
             "#   rocprofv3 --kernel-trace --stats -f csv -d OUT -o run -- python3 bench.py %s" % bench_args,
             "# summary: python3 bench.py --stats-summary OUT/run_kernel_stats.csv %s" % bench_args]
    if op == "step":
        lines += ["# averages over every launch of the run: warm-up and the timed regions, whole steps (one",
                  "# launch per kernel over a group of layers, <..., 16>) and one-layer calls (<..., 1>)"]
    lines += ["",
             "%8s %12s %10s %10s %10s %7s  %s" % ("calls", "total ms", "avg us", "min us", "max us", "%", "kernel")]
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            lines.append("%8s %12.3f %10.2f %10.2f %10.2f %7.2f  %s" % (
                r["Calls"], float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"]), r["Name"][:110]))
    return "\n".join(lines) + "\n"


def read_pmc_summary(workload):
    path = pmc_file(workload)
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def read_traffic(workload, grouped):
    """The scoring kernel's measured HBM bytes per launch (of a group of
    layers, or of one layer), or None when there is no summary for this
    workload or the kernel changed since."""
    kv = read_pmc_summary(workload)
    key = "traffic_bytes_per_group_launch" if grouped else "traffic_bytes_per_layer_launch"
    if kv.get("source_sha256") != score_source_hash() or key not in kv:
        return None
    return int(kv[key])


def read_attn_traffic(workload):
    """The attention kernel's measured HBM bytes per launch over a group of
    layers, or None when there is no summary or the kernel changed since."""
    kv = read_pmc_summary(workload)
    key = "attn_traffic_bytes_per_group_launch"
    if kv.get("attn_source_sha256") != score_source_hash(ATTN_SOURCES) or key not in kv:
        return None
    return int(kv[key])


def h2d_copy_gbs(n_bytes=1 << 28, reps=10):
    """The PCIe reference measured on the same machine: a plain copy of a pinned
    host buffer to the GPU (the DMA engines), GB/s over `reps` copies."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return n_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


BENCH_STREAM_SRC = os.path.join(ROOT, "bench_stream.hip")
BENCH_STREAM_LIB = os.path.join(ROOT, "_build", "libqsabench.so")


def build_stream_probe():
    """Compile bench_stream.hip (the streaming-read reference) for gfx950."""
    import subprocess
    os.makedirs(os.path.dirname(BENCH_STREAM_LIB), exist_ok=True)
    tmp = BENCH_STREAM_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", BENCH_STREAM_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for bench_stream.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, BENCH_STREAM_LIB)
    return BENCH_STREAM_LIB


def stream_read_gbs(n_bytes=1660944384 // (1 << 20) * (1 << 20), reps=10):
    """GB/s of a plain front-to-back read of an n_bytes device buffer (256 KB
    per workgroup, eight 16-byte loads in flight per lane), timed with events
    over `reps` reads."""
    import torch
    if not os.path.exists(BENCH_STREAM_LIB):
        raise RuntimeError("libqsabench.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(BENCH_STREAM_LIB)
    lib.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.bench_stream_read.restype = ctypes.c_int
    chunk = 256 * 1024
    n_wg = n_bytes // chunk
    buf = torch.empty(n_wg * chunk, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        if lib.bench_stream_read(ctypes.c_void_p(buf.data_ptr()), n_wg, chunk, ctypes.c_void_p(out.data_ptr()), s):
            raise RuntimeError("bench_stream_read failed")

    for _ in range(3):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return n_wg * chunk * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def stream_ceiling(step_gbs, scan_gbs):
    """A streaming-read ceiling measured on the same GPU: a plain read of a
    buffer the size of the 12-layer index (1.66 GB). The step's and the
    scan's algorithmic GB/s are given as fractions of it."""
    gbs = stream_read_gbs()
    return {"achieved": round(gbs, 1), "unit": "GB/s", "kind": "plain streaming read of 1.66 GB",
            "step_frac": round(step_gbs / gbs, 4), "scan_frac": round(scan_gbs / gbs, 4)}


def ctx_label(n):
    """262144 -> '256K', 1048576 -> '1M'."""
    if n % (1 << 20) == 0:
        return "%dM" % (n >> 20)
    if n % 1024 == 0:
        return "%dK" % (n >> 10)
    return str(n)


def metric_for(wl, kv_host):
    """The metric string of a workload's decode step (the headline workload's
    is the one the reference's benchmark is quoted with)."""
    if wl.ctx is not None and len(set(wl.ctx)) == 1:
        size = "%d\u00d7%s" % (wl.batch, ctx_label(int(wl.ctx[0])))
    elif wl.ctx is not None:
        size = "%d sequences of %s-%s" % (wl.batch, ctx_label(min(wl.ctx)), ctx_label(max(wl.ctx)))
    else:
        size = "%d\u00d7U[%d,%d]" % (wl.batch, wl.ragged[0], wl.ragged[1])
    if kv_host:
        return "QSA decode layer-steps/s at %s ctx, KV in pinned host memory; achieved PCIe GB/s as %% of peak" % size
    return "QSA decode layer-steps/s at %s ctx; achieved HBM GB/s as %% of peak" % size


def step_percentiles(ms):
    """p10 / median / p90 (and the extremes) of per-step times in ms."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "median": round(float(np.median(a)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "min": round(float(a.min()), 4),
            "max": round(float(a.max()), 4), "n": int(a.size)}


def timed_region(run, n, stream):
    """Runs `run()` n times back to back between two events, with nothing
    recorded and no synchronisation inside the region: the mean per call in
    ms."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def timed_steps(run, n, stream):
    """The per-call times of n calls with an event between consecutive calls,
    then the mean of n more calls timed as one region (timed_region). An
    event recorded after a call delays the next one by 1.5-3 us, so the
    first run gives the spread of the calls and the second their mean; the
    first also carries the first calls after the warm-up, which run slower."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    mean = timed_region(run, n, stream)
    return mean, per


def copy_calibration():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copies": 3}), flush=True)


class HipEvents:
    """hipEvent_t through the HIP runtime already loaded in this process."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.rt = ctypes.CDLL(path)
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        return e.value


    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def recorded(self, a, b):
        """Whether the pair (a, b) has been recorded: the elapsed time of a
        pair that never was is an error."""
        ms = ctypes.c_float()
        ok = self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        if not ok:
            self.rt.hipGetLastError()            # clear it, so that no later check reports it
        return ok


def tokens_selected(sel, ns, ctx):
    """Tokens covered by each (layer, sequence) selection (host arithmetic)."""
    import numpy as np
    L, B, _ = sel.shape
    out = np.zeros((L, B), np.int64)
    for l in range(L):
        for b in range(B):
            n = int(ns[l, b])
            if n == 0:
                continue
            last = int(sel[l, b, n - 1])
            out[l, b] = 4 * (n - 1) + min(4, int(ctx[b]) - 4 * last)
    return out


def cpu_baseline(wl, hi, seconds):
    """The oracle, single-threaded, on (layer, sequence) units of the workload
    taken in order (layer 0's sequences first) until about `seconds` of oracle
    time have run. Input generation (the host C generator) is excluded.
    Returns layer-steps/s = 1 / (batch * mean unit time)."""
    import numpy as np
    import oracle
    import qsa_synth as S
    from qsa_synth import host as SH
    g = S.GEOM
    K = wl.budget // g.block_tokens
    times, units = [], []
    for l in range(wl.layers):
        for b in range(wl.batch):
            if sum(times) >= seconds:
                break
            L = int(hi.lay.ctx[b])
            keys, sig = SH.index_keys(wl.seed, l, b, 0, L, hi.lay.planted[(l, b)], hi.u[l, b])
            t0 = time.perf_counter()
            ts = oracle.token_scores(keys, sig, hi.q_idx[l, b], hi.w[l, b])
            bs = oracle.block_scores(ts, g.block_tokens)
            sel = oracle.select_blocks(bs, K, oracle.forced_mask(L, g.block_tokens, wl.sink_blocks, wl.tail_tokens))
            toks = oracle.tokens_of_blocks(L, sel.blocks, g.block_tokens)
            t1 = time.perf_counter()
            rows = SH.kv_rows(wl.seed, l, hi.lay.pt[b, toks])          # input generation, not timed
            t2 = time.perf_counter()
            oracle.attention(np.arange(len(toks)), None, rows, hi.q[l, b], g.n_kv_heads, g.sm_scale)
            t3 = time.perf_counter()
            times.append((t1 - t0) + (t3 - t2))
            units.append((l, b))
    mean = sum(times) / len(times)
    single = {"value": 1.0 / (wl.batch * mean), "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
              "sample": "%d (layer, sequence) units of %s (layers %d-%d, %.1f s of oracle time), single-threaded "
                        "C oracle in fp64: %.3f s per unit, and a layer-step is %d units; input generation excluded"
                        % (len(units), wl.name, units[0][0], units[-1][0], sum(times), mean, wl.batch)}

    # All host cores (at most 16, one GPU's share of the host): one thread per
    # core, each running the oracle on its own (layer, sequence) unit over and
    # over for about seconds / 2. The C oracle and the generator release the
    # GIL, so the threads run in parallel; inputs are generated before timing.
    import threading
    n_thr = max(1, min(16, len(os.sched_getaffinity(0))))
    all_units = [(l, b) for l in range(wl.layers) for b in range(wl.batch)]
    picked = [all_units[i % len(all_units)] for i in range(n_thr)]
    inputs = []
    for (l, b) in picked:
        L = int(hi.lay.ctx[b])
        keys, sig = SH.index_keys(wl.seed, l, b, 0, L, hi.lay.planted[(l, b)], hi.u[l, b])
        inputs.append((l, b, L, keys, sig))
    done = [0] * n_thr
    t_start = [0.0]
    ready = threading.Barrier(n_thr + 1)
    go = threading.Barrier(n_thr + 1)

    def work(i):
        try:
            run(i)
        except BaseException:
            ready.abort()                           # no thread waits forever on a failed one
            go.abort()
            raise

    def run(i):
        l, b, L, keys, sig = inputs[i]

        def select():
            ts = oracle.token_scores(keys, sig, hi.q_idx[l, b], hi.w[l, b])
            bs = oracle.block_scores(ts, g.block_tokens)
            sel = oracle.select_blocks(bs, K, oracle.forced_mask(L, g.block_tokens, wl.sink_blocks, wl.tail_tokens))
            return oracle.tokens_of_blocks(L, sel.blocks, g.block_tokens)

        # untimed: the unit's rows (its selection is the same every time)
        rows = SH.kv_rows(wl.seed, l, hi.lay.pt[b, select()])
        ready.wait()
        go.wait()
        while time.perf_counter() < t_start[0] + seconds / 2:
            toks = select()
            oracle.attention(np.arange(len(toks)), None, rows, hi.q[l, b], g.n_kv_heads, g.sm_scale)
            done[i] += 1

    thr = [threading.Thread(target=work, args=(i,)) for i in range(n_thr)]
    for t in thr:
        t.start()
    try:
        ready.wait()
        t_start[0] = time.perf_counter()
        go.wait()
    except threading.BrokenBarrierError:
        pass
    for t in thr:
        t.join()
    if ready.broken or go.broken:
        return single
    wall = time.perf_counter() - t_start[0]
    n_done = sum(done)
    if n_done == 0:
        return single
    return {"value": n_done / wall / wl.batch, "unit": "layer-steps/s", "cores": n_thr, "kind": "oracle",
            "sample": "%d threads (one per host core, at most 16), each running the C oracle (fp64) on its own "
                      "(layer, sequence) unit of %s over and over: %d units in %.1f s of wall time, and a "
                      "layer-step is %d units; input generation excluded" % (n_thr, wl.name, n_done, wall,
                                                                            wl.batch),
            "single_core": single}


def context_sweep(args, known):
    """The headline schedule at a fixed budget over three contexts (8 x 16K,
    64K and 256K tokens, 12 layers): the step time, the scan launch's time
    (HIP events taken by the launch) and what is left, the selection chain
    and attention, which do not grow with the context. `known` holds the
    headline workload's (ms_per_step, scan_ms), measured already."""
    import numpy as np
    import torch
    import kv_cache_selection_amd as qsa
    import qsa_synth as S
    from qsa_synth.device import DeviceInputs
    g = S.GEOM
    dev = torch.device("cuda:0")
    hev = HipEvents()
    points = []
    for name in ("batch8-16k", "batch8-64k", "batch8-256k"):
        wl = S.WORKLOADS[name]
        if name in known:
            ms, scan_ms = known[name]
        else:
            di = DeviceInputs(wl, dev)
            NL, B = di.n_layers, di.batch
            K = wl.budget // g.block_tokens
            cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, g.sm_scale)
            bt = qsa.make_batch(B, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
            sel = torch.zeros((NL, B, K), dtype=torch.int32, device=dev)
            ns = torch.zeros((NL, B), dtype=torch.int32, device=dev)
            nws = qsa.qsa_workspace_size(cfg, B, di.max_ctx, NL, qsa.QSA_KV_DEVICE)
            ws = torch.empty(nws, dtype=torch.uint8, device=dev)
            stream = torch.cuda.current_stream()
            side = [torch.cuda.Stream()]
            events = qsa.StepEvents(NL, 1)
            ev = (hev.create(), hev.create())
            lys = [qsa.make_layer(di.keys[l], di.scales[l], di.q_idx[l], di.w_idx[l], di.q[l], di.pool[l],
                                  di.out[l], None, sel[l], ns[l], ev if l == 0 else None) for l in range(NL)]

            def run():
                qsa.qsa_decode_step(cfg, bt, lys, qsa.QSA_KV_DEVICE, ws, nws, stream, side, events)

            for _ in range(args.warmup):
                run()
            ms, _ = timed_steps(run, args.steps, stream)
            scans = []
            for _ in range(args.steps):
                run()
                torch.cuda.synchronize()
                scans.append(hev.elapsed_ms(*ev))
            scan_ms = float(np.mean(scans))
            del di, ws, lys
            torch.cuda.empty_cache()
        ctx = int(wl.ctx[0])
        idx_bytes = wl.batch * ctx * g.index_row_bytes * wl.layers
        points.append({"workload": name, "ctx": ctx, "ms_per_step": round(ms, 4),
                       "scan_us": round(scan_ms * 1e3, 2), "non_scan_us": round((ms - scan_ms) * 1e3, 2),
                       "scan_gbs": round(idx_bytes / (scan_ms * 1e-3) / 1e9, 1)})
    return {"budget_tokens": 2048, "batch": 8, "layers": 12, "points": points,
            "note": "non_scan_us = step - scan launch: selection chain, attention over the 2048 selected tokens "
                    "per sequence and layer, merge, launch gaps"}


def bench_append(args):
    """The append step alone: one token enters every layer of every sequence
    (quantised index row, KV row, page-table entry). The lengths are not
    advanced, so every timed call does the same work."""
    import numpy as np
    import torch
    import kv_cache_selection_amd as qsa
    import qsa_synth as S
    g = S.GEOM
    wl = S.WORKLOADS[args.workload]
    B, NL = wl.batch, wl.layers
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(wl.seed)
    ctx = (np.array(S.ctx_lengths(wl)) // 2).astype(np.int32)     # the new token lands mid-sequence
    cap = ctx + 1
    row0 = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    n_rows, stride = int(cap.sum()), int(cap.max())
    n_slots = 1 << 16
    d_ctx = torch.from_numpy(ctx).to(dev)
    d_row0 = torch.from_numpy(row0).to(dev)
    d_pt = torch.zeros((B, stride), dtype=torch.int32, device=dev)
    keys = [torch.zeros((n_rows, g.idx_dim), dtype=torch.uint8, device=dev) for _ in range(NL)]
    scales = [torch.zeros(n_rows, dtype=torch.int16, device=dev) for _ in range(NL)]
    pools = [torch.zeros((n_slots, g.row_elems), dtype=torch.int16, device=dev) for _ in range(NL)]
    new_keys = [torch.from_numpy(rng.standard_normal((B, g.idx_dim)).astype(np.float32)).to(dev) for _ in range(NL)]
    new_rows = [torch.from_numpy(rng.integers(-2 ** 15, 2 ** 15, (B, g.row_elems)).astype(np.int16)).to(dev)
                for _ in range(NL)]
    slots = torch.from_numpy(rng.choice(n_slots, B, replace=False).astype(np.int32)).to(dev)
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, g.sm_scale)
    bt = qsa.make_batch(B, stride, d_ctx, d_row0, d_pt, stride, n_slots, n_rows)
    lys = [qsa.make_append_layer(new_keys[l], new_rows[l], keys[l], scales[l], pools[l]) for l in range(NL)]
    stream = torch.cuda.current_stream()

    def call():
        qsa.qsa_append_token(cfg, bt, lys, qsa.QSA_KV_DEVICE, slots, d_pt, None, stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    # bytes the step must move: read the fp32 key and the bf16 row, write the
    # 64 codes + 2-byte scale and the 2048-byte row, per sequence and layer
    per = g.idx_dim * 4 + g.row_bytes + g.idx_dim + 2 + g.row_bytes
    moved = B * NL * per + B * 4
    gbs = moved / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "QSA append step: tokens entered into every QSA layer's cache per second",
        "value": round(B / (us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "us_per_call": round(us, 3), "higher_is_better": True,
        "dtype": "f32 key -> e4m3+f16 scale; bf16 row copy", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "layers": NL, "op": "append"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 6), "bytes_per_call": moved,
                     "note": "one wavefront per sequence; the call is launch- and latency-bound"},
    }), flush=True)


def bench_lease(args):
    """Slot leases: the host pool's throughput, and the two device calls that
    go with it -- the generation check over a whole batch (a bandwidth-bound
    scan of the page table and token generations) and a ring spill move."""
    import numpy as np
    import torch
    import kv_cache_selection_amd as qsa
    import qsa_synth as S
    g = S.GEOM
    wl = S.WORKLOADS[args.workload]
    B, NL = wl.batch, wl.layers
    dev = torch.device("cuda:0")
    # host pool: 8 leases with a 64-slot tail ring, 4096 tokens each, then closed
    pool = qsa.SlotPool(B * 4096 + B * 64)
    t0 = time.perf_counter()
    leases = [pool.open(64) for _ in range(B)]
    n_ops = 0
    for _ in range(4096):
        for lid in leases:
            pool.next_token(lid)
            n_ops += 1
    for lid in leases:
        pool.close(lid)
    host_s = time.perf_counter() - t0
    assert pool.free_slots() == pool.n_slots
    # generation check at the workload's full size
    ctx = np.array(S.ctx_lengths(wl), np.int32)
    stride = int(ctx.max())
    n_slots = int(ctx.sum())
    rng = np.random.default_rng(wl.seed)
    perm = rng.permutation(n_slots).astype(np.int32)
    pt = np.full((B, stride), -1, np.int32)
    off = 0
    for b in range(B):
        pt[b, :ctx[b]] = perm[off:off + ctx[b]]
        off += ctx[b]
    slot_gen = rng.integers(0, 1 << 20, n_slots).astype(np.uint32)
    tok_gen = np.where(pt >= 0, slot_gen[np.maximum(pt, 0)], 0).astype(np.uint32)
    d_ctx = torch.from_numpy(ctx).to(dev)
    d_pt = torch.from_numpy(pt).to(dev)
    d_tg = torch.from_numpy(tok_gen.view(np.int32)).to(dev)
    d_sg = torch.from_numpy(slot_gen.view(np.int32)).to(dev)
    stale = torch.zeros(B, dtype=torch.int32, device=dev)
    bt = qsa.make_batch(B, stride, d_ctx, torch.zeros(B, dtype=torch.int64, device=dev), d_pt, stride, n_slots, 0)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        qsa.qsa_check_generations(bt, d_pt, d_tg, d_sg, stale, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        qsa.qsa_check_generations(bt, d_pt, d_tg, d_sg, stale, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    check_us = e0.elapsed_time(e1) / args.steps * 1e3
    assert int(stale.sum()) == 0
    check_bytes = int(ctx.sum()) * 12          # page-table entry + token generation + slot generation
    check_gbs = check_bytes / (check_us * 1e-6) / 1e9
    # a ring spill: one token per sequence moves in every layer's pool
    pools = [torch.zeros((1 << 16, g.row_elems), dtype=torch.int16, device=dev) for _ in range(NL)]
    mpt = torch.from_numpy(rng.permutation(1 << 16)[:B * 64].reshape(B, 64).astype(np.int32)).to(dev)
    mb = qsa.make_batch(B, 64, d_ctx, torch.zeros(B, dtype=torch.int64, device=dev), mpt, 64, 1 << 16, 0)
    tok = torch.full((B,), 5, dtype=torch.int64, device=dev)
    dst = torch.from_numpy(rng.permutation(1 << 16)[:B].astype(np.int32)).to(dev)
    for _ in range(args.warmup):
        qsa.qsa_move_tokens(mb, pools, qsa.QSA_KV_DEVICE, tok, dst, mpt, stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        qsa.qsa_move_tokens(mb, pools, qsa.QSA_KV_DEVICE, tok, dst, mpt, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    move_us = e0.elapsed_time(e1) / args.steps * 1e3
    print(json.dumps({
        "metric": "QSA slot leases: generation check of a whole batch's page table",
        "value": round(int(ctx.sum()) / (check_us * 1e-6) / 1e9, 3), "unit": "G tokens checked/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "us_per_check": round(check_us, 2), "higher_is_better": True,
        "dtype": "int32 / uint32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "tokens": int(ctx.sum()), "op": "lease"},
        "roofline": {"bound": "hbm", "achieved": round(check_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(check_gbs / HBM_PEAK_GBS, 4), "bytes_per_check": check_bytes},
        "move_tokens_us": round(move_us, 2),
        "host_pool": {"ops_per_s": round(n_ops / host_s), "ops": n_ops,
                      "note": "open + next_token + close through ctypes, one host thread"},
    }), flush=True)


def bench_multi(args):
    """Multi-query scoring (prefill / chunked decode): n_queries causal queries
    per sequence, the chunk of positions at the end of each sequence, over the
    workload's index (one layer)."""
    import numpy as np
    import torch
    import kv_cache_selection_amd as qsa
    import qsa_synth as S
    from qsa_synth.device import DeviceInputs
    g = S.GEOM
    wl = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    di = DeviceInputs(wl, dev, layers=1, kv_host=False)
    B, Q = di.batch, args.queries
    rng = np.random.default_rng(wl.seed)
    ctx = di.hi.lay.ctx
    pos = np.stack([np.arange(int(ctx[b]) - Q, int(ctx[b])) for b in range(B)]).astype(np.int32)
    q_idx = torch.from_numpy(S.f32_to_bf16_bits(rng.standard_normal((B, Q, g.idx_heads, g.idx_dim))
                                                .astype(np.float32)).view(np.int16)).to(dev)
    w = torch.from_numpy(rng.uniform(0, 1, (B, Q, g.idx_heads)).astype(np.float32)).to(dev)
    d_pos = torch.from_numpy(pos).to(dev)
    nb = (di.max_ctx + 3) // 4
    out = torch.empty((B, Q, nb), dtype=torch.float32, device=dev)
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, g.sm_scale)
    bt = qsa.make_batch(B, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    stream = torch.cuda.current_stream()

    def call():
        qsa.qsa_index_score_multi(cfg, bt, Q, di.keys[0], di.scales[0], q_idx, w, d_pos, out, nb, stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    tokens = int(ctx.sum())
    moved = tokens * (g.index_row_bytes + Q)                  # index read + Q/4 fp32 block scores per token
    flops = tokens * 512 * Q                                  # 4 heads x 64 dims x 2, per query and token
    lane_ops = tokens * 9 * Q                                 # per query-token: 4 ReLU, 4 weight fma, 1 scale
    gbs = moved / (us * 1e-6) / 1e9
    tfs = flops / (us * 1e-6) / 1e12
    tops = lane_ops / (us * 1e-6) / 1e12
    mfma_peak = 2500.0                                        # dense bf16 TFLOP/s
    valu_peak = 256 * 4 * 16 * 2.4e9 / 1e12                   # fp32 lane-ops/s without packed math: 39.3 T
    hbm_bound = gbs / HBM_PEAK_GBS >= tfs / mfma_peak
    print(json.dumps({
        "metric": "QSA multi-query index scoring: query-token scores per second",
        "value": round(tokens * Q / (us * 1e-6) / 1e9, 2), "unit": "G query-token scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "us_per_launch": round(us, 2), "higher_is_better": True,
        "dtype": "fp8e4m3 keys, bf16 queries, fp32 accumulate", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "ctx": int(ctx.max()), "queries": Q, "op": "multi"},
        "roofline": ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": moved}
                     if hbm_bound else
                     {"bound": "mfma", "achieved": round(tfs, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                      "frac": round(tfs / mfma_peak, 4), "flops_per_launch": flops}),
        "mfma": {"achieved": round(tfs, 1), "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(tfs / mfma_peak, 4)},
        "valu": {"achieved": round(tops, 2), "peak": round(valu_peak, 1), "unit": "T fp32 lane-ops/s",
                 "frac": round(tops / valu_peak, 4), "lane_ops_per_launch": lane_ops},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="batch8-256k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time spent on the CPU baseline (0: skip)")
    ap.add_argument("--side-streams", type=int, default=None,
                    help="side streams of the overlapped schedule (default: 1, or 3 with a hot cache); 0: every "
                         "kernel in order on one stream")
    ap.add_argument("--op", choices=("step", "append", "lease", "multi"), default="step",
                    help="step: the decode step (default); append: the append step alone; lease: slot leases; "
                         "multi: multi-query scoring")
    ap.add_argument("--queries", type=int, default=64, help="queries per sequence for --op multi")
    ap.add_argument("--no-sweep", dest="sweep", action="store_false",
                    help="skip the fixed-budget context sweep (8 x {16K, 64K, 256K})")
    ap.add_argument("--copy-calibration", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--pmc-summary", nargs=4, metavar="CSV", help=argparse.SUPPRESS)
    ap.add_argument("--stats-summary", metavar="CSV", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.stats_summary:
        extra = [a for a in sys.argv[1:] if a not in ("--stats-summary", args.stats_summary)]
        sys.stdout.write(stats_summary(args.stats_summary, args.workload, args.op, " ".join(extra)))
        return
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(args.pmc_summary, args.workload))
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: libqsa runs the QSA decode step on a single MI355X and has no "
              "multi-GPU path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.op == "append":
        bench_append(args)
        return
    if args.op == "lease":
        bench_lease(args)
        return
    if args.op == "multi":
        bench_multi(args)
        return

    import numpy as np
    import torch

    import kv_cache_selection_amd as qsa
    import qsa_synth as S
    from qsa_synth.device import DeviceInputs

    wl = S.WORKLOADS[args.workload]
    g = S.GEOM
    dev = torch.device("cuda:0")
    t_setup = time.time()
    di = DeviceInputs(wl, dev)
    print("[bench] inputs resident in %.1f s" % (time.time() - t_setup), file=sys.stderr, flush=True)

    loc = qsa.QSA_KV_HOST_PINNED if di.kv_host else qsa.QSA_KV_DEVICE
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, g.sm_scale)
    bt = qsa.make_batch(di.batch, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    K = wl.budget // g.block_tokens
    NL = di.n_layers
    sel = torch.zeros((NL, di.batch, K), dtype=torch.int32, device=dev)
    ns = torch.zeros((NL, di.batch), dtype=torch.int32, device=dev)
    nws = qsa.qsa_workspace_size(cfg, di.batch, di.max_ctx, NL, loc)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # the second scan stream (HBM pools), the PCIe gather (host pools) or the
    # per-layer chains (hot cache) run on side streams
    if args.side_streams is None:
        args.side_streams = 3 if wl.hot_slots else 1
    side = [torch.cuda.Stream() for _ in range(args.side_streams)]
    events = qsa.StepEvents(NL, len(side)) if side else None

    # Workloads that run many decode steps cycle through step_variants query
    # sets (drifting indexer queries); the others repeat one step.
    NV = max(1, wl.step_variants)
    qv = []
    for v in range(NV if NV > 1 else 0):
        qi, qq = S.step_queries(wl, di.hi, v)
        qv.append((torch.from_numpy(qi.view(np.int16)).to(dev), torch.from_numpy(qq.view(np.int16)).to(dev)))
    hot, n_miss = None, None
    if wl.hot_slots:
        H = wl.hot_slots
        n_miss = torch.zeros((NL, di.batch), dtype=torch.int32, device=dev)
        hot = []
        for l in range(NL):
            hc = qsa.make_hot_cache(torch.zeros((di.batch, H, g.row_elems), dtype=torch.int16, device=dev),
                                    torch.zeros((di.batch, di.pt_stride), dtype=torch.int32, device=dev),
                                    torch.zeros((di.batch, H), dtype=torch.int32, device=dev), H, n_miss[l])
            qsa.qsa_hot_reset(bt, hc)
            hot.append(hc)

    def layers(v=0, events=None):
        return [qsa.make_layer(di.keys[l], di.scales[l], qv[v][0][l] if qv else di.q_idx[l], di.w_idx[l],
                               qv[v][1][l] if qv else di.q[l], di.pool[l], di.out[l], None, sel[l], ns[l],
                               events[l] if events else None, hot[l] if hot else None) for l in range(NL)]

    plain = [layers(v) for v in range(NV)]
    n_done = [0]

    def step(lys, streams=True):
        qsa.qsa_decode_step(cfg, bt, lys[n_done[0] % NV], loc, ws, nws, stream, side if streams else None,
                            events if streams else None)
        n_done[0] += 1

    for _ in range(args.warmup):
        step(plain)
    torch.cuda.synchronize()

    # Timed region 1: whole steps, an event between consecutive steps.
    ms_step, per_step = timed_steps(lambda: step(plain), args.steps, stream)
    ctx = di.hi.lay.ctx
    ntok = tokens_selected(sel.cpu().numpy(), ns.cpu().numpy(), ctx)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Timed region 1b (HBM workloads with one query set): the same steps with
    # drifting indexer queries, cycling through DRIFT_VARIANTS query sets so
    # that consecutive steps select different (overlapping) rows and no step
    # re-reads exactly the rows the one before it read.
    drifting = None
    if NV == 1 and not di.kv_host and not hot:
        import dataclasses
        wl_d = dataclasses.replace(wl, drift=DRIFT, step_variants=DRIFT_VARIANTS)
        qd = []
        for v in range(DRIFT_VARIANTS):
            qi, qq = S.step_queries(wl_d, di.hi, v)
            qd.append((torch.from_numpy(qi.view(np.int16)).to(dev), torch.from_numpy(qq.view(np.int16)).to(dev)))
        dl = [[qsa.make_layer(di.keys[l], di.scales[l], qd[v][0][l], di.w_idx[l], qd[v][1][l], di.pool[l],
                              di.out[l], None, sel[l], ns[l]) for l in range(NL)] for v in range(DRIFT_VARIANTS)]
        # the blocks that consecutive query sets share (untimed)
        sels = []
        for v in range(DRIFT_VARIANTS):
            qsa.qsa_decode_step(cfg, bt, dl[v], loc, ws, nws, stream, side, events)
            torch.cuda.synchronize()
            sels.append((sel.cpu().numpy().copy(), ns.cpu().numpy().copy()))
        shared = []
        for v in range(DRIFT_VARIANTS):
            (a, na), (b, nb) = sels[v], sels[(v + 1) % DRIFT_VARIANTS]
            for l in range(NL):
                for q in range(di.batch):
                    sa, sb = set(a[l, q, :na[l, q]].tolist()), set(b[l, q, :nb[l, q]].tolist())
                    shared.append(len(sa & sb) / max(len(sa), 1))
        k_d = [0]

        def step_drift():
            qsa.qsa_decode_step(cfg, bt, dl[k_d[0] % DRIFT_VARIANTS], loc, ws, nws, stream, side, events)
            k_d[0] += 1

        for _ in range(args.warmup):
            step_drift()
        ms_drift, per_drift = timed_steps(step_drift, args.steps, stream)
        drifting = {"ms_per_step": round(ms_drift, 4), "value": round(NL / (ms_drift * 1e-3), 2),
                    "step_ms": step_percentiles(per_drift), "query_variants": DRIFT_VARIANTS, "drift": DRIFT,
                    "shared_blocks_consecutive": round(float(np.mean(shared)), 4),
                    "note": "indexer queries bf16(q_idx + drift N(0,1)), a new draw per variant, and fresh "
                            "attention queries; the variants are cycled, so consecutive steps select overlapping "
                            "but different blocks"}

    # Timed region 1c (HBM workloads): each step timed alone after a read of
    # COLD_FLUSH_BYTES of another buffer, twice the 256 MB Infinity Cache, so
    # that nothing an earlier step read is left in it. Against region 1's
    # per-step times this shows what the steps gain from that cache.
    cold = None
    if not di.kv_host:
        flush = torch.ones(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        n_cold = min(args.steps, 20)
        ev_c = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
        sink = torch.zeros((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for i in range(n_cold):
            sink += flush.sum()
            ev_c[i][0].record(stream)
            step(plain)
            ev_c[i][1].record(stream)
        torch.cuda.synchronize()
        per_cold = [a.elapsed_time(b) for a, b in ev_c]
        del flush
        cold = {"step_ms": step_percentiles(per_cold), "flush_bytes": COLD_FLUSH_BYTES,
                "median_over_warm": round(float(np.median(per_cold) / np.median(per_step)), 4),
                "note": "each step timed alone after reading a separate buffer of flush_bytes (twice the "
                        "Infinity Cache); median_over_warm compares with the back-to-back steps of step_ms"}

    # Timed region 2: the same steps with no side stream (everything in order
    # on the compute stream).
    ms_serial = None
    if side:
        e0.record(stream)
        for _ in range(args.steps):
            step(plain, streams=False)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_serial = e0.elapsed_time(e1) / args.steps

    # Timed region 2b: a step as a model with dependent layers runs it, one
    # call per layer (n_layers = 1, one stream), each call with the
    # workspace a one-layer call needs.
    ms_per_layer_calls = None
    if not hot:
        nws1 = qsa.qsa_workspace_size(cfg, di.batch, di.max_ctx, 1, loc)
        ws1 = torch.empty(nws1, dtype=torch.uint8, device=dev)

        def step_per_layer():
            lys = plain[n_done[0] % NV]
            for ly in lys:
                qsa.qsa_decode_step(cfg, bt, [ly], loc, ws1, nws1, stream, None)
            n_done[0] += 1

        step_per_layer()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step_per_layer()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_layer_calls = e0.elapsed_time(e1) / args.steps

    # Timed region 3: the headline schedule again, with HIP events around
    # the scoring launches. A launch that scans a group of layers takes the
    # events of the group's first layer, so only those are recorded: with
    # HBM pools one launch scans all the layers (up to 16), the pinned-host
    # pipeline scans groups of 1, 2, 4, ... layers, and the one-stream
    # schedule scans layer by layer. The roofline is the scanned bytes over
    # the scan launches' summed durations.
    hev = HipEvents()
    evs = [(hev.create(), hev.create()) for _ in range(NL)]
    timed = [layers(v, evs) for v in range(NV)]
    step(timed)                          # which layers lead a scan launch
    torch.cuda.synchronize()
    ev_used = [p for p in evs if hev.recorded(*p)]
    durs = []
    for _ in range(args.steps):
        step(timed)
        torch.cuda.synchronize()
        durs.append(sum(hev.elapsed_ms(a, b) for (a, b) in ev_used))
    n_launch = len(ev_used)
    score_ms = float(np.mean(durs)) / n_launch             # per launch
    layers_per_launch = NL / n_launch

    # Timed region 4: every one-layer scoring launch timed alone, as a
    # kernel-trace profile sees it: the one-layer calls of region 2b (the
    # one-stream step with a hot cache, which runs layer by layer).
    durs1 = []
    timed1 = [layers(v, evs) for v in range(NV)]
    for _ in range(args.steps):
        if hot:
            step(timed1, streams=False)
        else:
            for ly in timed1[n_done[0] % NV]:
                qsa.qsa_decode_step(cfg, bt, [ly], loc, ws1, nws1, stream, None)
            n_done[0] += 1
        torch.cuda.synchronize()
        durs1.extend(hev.elapsed_ms(a, b) for (a, b) in evs)
    score1_ms = float(np.mean(durs1))

    # Hot cache: rows fetched over PCIe per step, over one cycle of the query
    # variants in the cache's steady state (untimed).
    fetched = None
    if hot:
        tot = 0
        for _ in range(NV):
            step(plain)
            torch.cuda.synchronize()
            tot += int(n_miss.sum())
        fetched = tot / NV

    idx_bytes_layer = int(ctx.sum()) * g.index_row_bytes
    idx_bytes_launch = int(round(idx_bytes_layer * layers_per_launch))
    step_bytes = idx_bytes_layer * NL + int(ntok.sum()) * g.row_bytes
    achieved = idx_bytes_launch / (score_ms * 1e-3) / 1e9
    achieved1 = idx_bytes_layer / (score1_ms * 1e-3) / 1e9
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    value = NL / (ms_step * 1e-3)

    rows_bytes = int(ntok.sum()) * g.row_bytes
    attn_traffic = read_attn_traffic(wl.name) if n_launch == 1 else None
    result = {
        "metric": metric_for(wl, di.kv_host),
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": step_percentiles(per_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16 in, fp32 accumulate",
        "data": "synthetic (seeded SplitMix64 generator; planted relevant blocks)",
        "config": {"workload": wl.name, "batch": wl.batch, "ctx": int(ctx.max()), "layers": NL,
                   "budget_tokens": wl.budget, "sink_blocks": wl.sink_blocks, "tail_tokens": wl.tail_tokens,
                   "kv": "host-pinned" if di.kv_host else "hbm", "side_streams": len(side),
                   "hot_cache_rows": wl.hot_slots},
        "roofline": {"bound": "hbm", "kernel": "index_score_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (read_traffic(wl.name, True) if n_launch == 1 else
                                 read_traffic(wl.name, False) if n_launch == NL else None),
                     "bytes_per_launch": idx_bytes_launch,
                     "layers_per_launch": round(layers_per_launch, 3), "launches_per_step": n_launch,
                     "avg_launch_us": round(score_ms * 1e3, 2)},
        # the scoring launch of a one-layer call, each launch alone
        "one_stream_score": {"achieved": round(achieved1, 1), "unit": "GB/s",
                             "frac": round(achieved1 / HBM_PEAK_GBS, 4), "bytes_per_launch": idx_bytes_layer,
                             "avg_launch_us": round(score1_ms * 1e3, 2),
                             "traffic": read_traffic(wl.name, False)},
        "per_layer_calls": None if ms_per_layer_calls is None else {
            "ms_per_step": round(ms_per_layer_calls, 4), "value": round(NL / (ms_per_layer_calls * 1e-3), 2),
            "note": "one qsa_decode_step call per layer (n_layers = 1), one stream"},
        "one_stream": {"ms_per_step": round(ms_serial if ms_serial is not None else ms_step, 4),
                       "value": round(NL / ((ms_serial if ms_serial is not None else ms_step) * 1e-3), 2)},
        # the whole step's index-scan + gathered-row bytes against the peak:
        # the fraction the target is stated in, and how far the step is from
        # 0.70 of it
        "step_hbm": {"achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes,
                     "target_frac": STEP_TARGET_FRAC,
                     "ms_at_target": round(step_bytes / (STEP_TARGET_FRAC * HBM_PEAK_GBS * 1e9) * 1e3, 4),
                     "shortfall_ms": round(ms_step - step_bytes / (STEP_TARGET_FRAC * HBM_PEAK_GBS * 1e9) * 1e3, 4)},
        # the attention launch of the headline schedule (all layers in one
        # launch): its algorithmic bytes (the selected rows) and the HBM
        # bytes the counters measured for it (profiles/), when current
        "attention": {"kernel": ATTN_KERNEL, "layers_per_launch": NL if n_launch == 1 else None,
                      "bytes_per_launch": rows_bytes if n_launch == 1 else None,
                      "traffic": attn_traffic,
                      "traffic_over_bytes": None if attn_traffic is None else round(attn_traffic / rows_bytes, 4)},
    }
    if drifting is not None:
        result["drifting"] = drifting
    if cold is not None:
        result["cold_cache"] = cold
    if di.kv_host:
        # every gathered row crosses PCIe once per step (with a hot cache: the misses only)
        pcie_bytes = int(ntok.sum()) * g.row_bytes if fetched is None else int(round(fetched)) * g.row_bytes
        pcie_gbs = pcie_bytes / (ms_step * 1e-3) / 1e9
        h2d = h2d_copy_gbs()
        result["pcie"] = {"achieved": round(pcie_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                          "frac": round(pcie_gbs / PCIE_PEAK_GBS, 4), "bytes_per_step": pcie_bytes,
                          "h2d_copy": round(h2d, 2), "frac_of_h2d_copy": round(pcie_gbs / h2d, 4)}
        if fetched is not None:
            result["hot_cache"] = {"rows_per_layer": wl.hot_slots, "drift": wl.drift, "query_variants": NV,
                                   "rows_fetched_per_step": round(fetched, 1),
                                   "rows_selected_per_step": int(ntok.sum()),
                                   "hit_rate": round(1.0 - fetched / max(int(ntok.sum()), 1), 4)}
    if not di.kv_host:
        result["stream_ceiling"] = stream_ceiling(step_gbs, achieved)
    if wl.name == "batch8-256k" and args.sweep:
        result["context_sweep"] = context_sweep(args, {wl.name: (ms_step, score_ms)})
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(wl, di.hi, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
