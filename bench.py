#!/usr/bin/env python3
"""Benchmark of the QSA sparse-attention decode step on one MI355X.

Workload (default): 8 sequences x 262,144 cached tokens, 12 QSA layers,
indexer_budget 2048 (512 C4 blocks), first block forced as a sink, 32 planted
relevant blocks per sequence per layer; index keys (66 B/token/layer) and the
bf16 KV pools (2048 B/token/layer, 51.5 GB) are resident in HBM before timing.
A step is one full pass of the hot path over all 12 layers (score -> select ->
paged attention -> merge) through the C ABI; the metric is layer-steps/s.

Prints one JSON line with the driver's fields plus:
  roofline      the dominant kernel (index scoring): algorithmic bytes per
                launch / its average duration, timed with HIP events recorded
                on the compute stream around each scoring launch;
  step_hbm      the whole step's algorithmic bytes (index scan + gathered
                rows) over the step time, against the same HBM peak;
  cpu_baseline  the CPU oracle, single-threaded, on a sample of (layer,
                sequence) units of the same workload, scaled to layer-steps/s.
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


def cpu_baseline(wl, hi, units):
    """Oracle time per (layer, sequence) unit, single thread; input generation
    excluded. Returns layer-steps/s = 1 / (batch * mean unit time)."""
    import numpy as np
    import oracle
    import qsa_synth as S
    g = S.GEOM
    K = wl.budget // g.block_tokens
    times = []
    for (l, b) in units:
        L = int(hi.lay.ctx[b])
        keys, sig = S.index_keys(wl.seed, l, b, 0, L, hi.lay.planted[(l, b)], hi.u[l, b])
        t0 = time.perf_counter()
        ts = oracle.token_scores(keys, sig, hi.q_idx[l, b], hi.w[l, b])
        bs = oracle.block_scores(ts, g.block_tokens)
        sel = oracle.select_blocks(bs, K, oracle.forced_mask(L, g.block_tokens, wl.sink_blocks, wl.tail_tokens))
        toks = oracle.tokens_of_blocks(L, sel.blocks, g.block_tokens)
        t1 = time.perf_counter()
        rows = S.kv_rows(wl.seed, l, hi.lay.pt[b, toks])          # input generation, not timed
        t2 = time.perf_counter()
        oracle.attention(np.arange(len(toks)), None, rows, hi.q[l, b], g.n_kv_heads, g.sm_scale)
        t3 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2))
    mean = sum(times) / len(times)
    return {"value": 1.0 / (wl.batch * mean), "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
            "sample": "%d (layer, sequence) units of %s (%s), single-threaded C oracle in fp64: "
                      "%.2f s per unit; a layer-step is %d units; input generation excluded"
                      % (len(units), wl.name, ", ".join("l%d/b%d" % u for u in units), mean, wl.batch)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="batch8-256k")
    ap.add_argument("--cpu-units", type=int, default=2, help="oracle units in the CPU baseline (0: skip)")
    ap.add_argument("--streams", type=int, default=2, choices=(1, 2),
                    help="2: overlap layers on a second stream (default); 1: every kernel in order on one stream")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the QSA decode step runs on a single MI355X and this build has "
              "no multi-GPU path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

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
    # select/attention (HBM pools) or the PCIe gather (host pools) overlap the scoring on a second stream
    copy = torch.cuda.Stream() if args.streams == 2 else None

    def layers(events=None):
        return [qsa.make_layer(di.keys[l], di.scales[l], di.q_idx[l], di.w_idx[l], di.q[l], di.pool[l], di.out[l],
                               None, sel[l], ns[l], events[l] if events else None) for l in range(NL)]

    plain = layers()

    def step(lys):
        qsa.qsa_decode_step(cfg, bt, lys, loc, ws, nws, stream, copy)

    for _ in range(args.warmup):
        step(plain)
    torch.cuda.synchronize()

    # Timed region 1: whole steps.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step(plain)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Timed region 2: the same steps with HIP events around every scoring launch.
    hev = HipEvents()
    evs = [(hev.create(), hev.create()) for _ in range(NL)]
    timed = layers(evs)
    durs = []
    for _ in range(args.steps):
        step(timed)
        torch.cuda.synchronize()
        durs.extend(hev.elapsed_ms(a, b) for (a, b) in evs)
    score_ms = float(np.mean(durs))

    ctx = di.hi.lay.ctx
    ntok = tokens_selected(sel.cpu().numpy(), ns.cpu().numpy(), ctx)
    idx_bytes_launch = int(ctx.sum()) * g.index_row_bytes
    step_bytes = idx_bytes_launch * NL + int(ntok.sum()) * g.row_bytes
    achieved = idx_bytes_launch / (score_ms * 1e-3) / 1e9
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    value = NL / (ms_step * 1e-3)

    result = {
        "metric": "QSA decode layer-steps/s at 8x256K ctx; achieved HBM GB/s as % of peak",
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16 in, fp32 accumulate",
        "data": "synthetic (seeded SplitMix64 generator; planted relevant blocks)",
        "config": {"workload": wl.name, "batch": wl.batch, "ctx": int(ctx.max()), "layers": NL,
                   "budget_tokens": wl.budget, "sink_blocks": wl.sink_blocks, "tail_tokens": wl.tail_tokens,
                   "kv": "host-pinned" if di.kv_host else "hbm", "streams": args.streams},
        "roofline": {"bound": "hbm", "kernel": "index_score_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": idx_bytes_launch,
                     "avg_launch_us": round(score_ms * 1e3, 2)},
        "step_hbm": {"achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes},
    }
    if args.cpu_units > 0:
        units = [(0, b) for b in range(min(args.cpu_units, wl.batch))]
        result["cpu_baseline"] = cpu_baseline(wl, di.hi, units)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
