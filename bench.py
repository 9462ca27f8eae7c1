"""Benchmark of split-KV grouped-query decode attention on one MI355X.

One step = one hipGraph replay of L layers x (partial kernel + combine kernel)
of the 28 query / 4 KV head, head_dim 128 decode shape (the 7B shape of
"10 · R4 — decode split-attention dim-parallel rewrite"), with every layer's
fp16 KV cache in its own buffer so that the 28 layers (1.9 GB at 32K context)
stream from HBM rather than from the 256 MB Infinity Cache. The live length is
set through positions[] on the device; the captured graph is the same for
every length.

Reported (one JSON line on stdout):
  value       KV-stream GB/s = algorithmic K+V bytes of the L layers / step time
              (the effective stream rate of "10 · R4", section 1)
  us/layer    step time / L (partial + combine + the gap between them)
  roofline    the partial kernel alone: K+V bytes per launch / its average
              duration, timed with HIP events on its own stream, against the
              8 TB/s HBM peak; `traffic` is the HBM bytes per launch measured by
              rocprofv3 counters (profiles/), or null when the counters were
              taken on another version of the kernel source
  cpu_baseline  the fp64 oracle on the host, one core, on one layer
  also        pct_of_probe (against the read stream measured on this GPU),
              total_bytes_per_layer / total_gbps (q, K+V, records written
              and read back, output)

Usage: python bench.py [--steps K] [--warmup W] [--nkv N] [--layers L]
       python bench.py --sweep          # split-count sweep, one line per point
       python bench.py --mode kernels   # eager partial/combine launches + a copy
       python bench.py --mode configs   # tiny / 7B@2K / hd256 workloads, warm+cold
       python bench.py --mode ragged    # 32-sequence ragged batch, split sweep
       python bench.py --mode oracle    # the fp64 oracle per workload (CPU only)
       python bench.py --mode step      # append + partial + combine per layer
       python bench.py --mode per_head --sweep-splits 18 36 64 128
                                        # grouped vs per-query-head grid
       python bench.py --mode rows      # n_q query rows per sequence (causal)
       python bench.py --mode long      # 28q/4kv hd128 at 16K..128K rows
       python bench.py --mode batch     # the same shape, 1..8 sequences at 16K/32K
       python bench.py --mode profile --workload growing|7b2k|hd256|ragged
                                        # one configuration's partial and
                                        # combine launches, for rocprofv3
       python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --kernels-json F
                                        # fold two rocprofv3 --pmc runs
       python bench.py --summarize-trace TRACE_DIR
                                        # per-layer partial / gap / combine
                                        # split of a --kernel-trace run
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV-stream GB/s (% of HBM peak) + µs/layer, 28q/4kv hd128 decode @2K–32K"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 1000 * 1000   # MI355X Infinity Cache (256 MB)
CSRC = os.path.join(ROOT, "decode_attention_gqa_amd", "csrc")
PARTIAL_SRCS = [os.path.join(CSRC, f) for f in (
    "splitkv_partial.hip", "splitkv_partial_mfma.hip",
    "splitkv_partial_common.h")]
COMBINE_SRCS = [os.path.join(CSRC, "splitkv_combine.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_hd128_g7_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths=PARTIAL_SRCS) -> str:
    """Hash of the kernel sources' code: comments and whitespace are removed
    first, so that editing a comment does not mark counters taken on the
    same code as stale."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
class Layers:
    """L layers of one decode shape, each layer's cache in its own buffers.

    Default: the 28q/4kv hd128 growing-context cache with per-block score
    offsets, max_ctx 33,024."""

    def __init__(self, layers: int, max_ctx: int, n_splits: int, block_len: int,
                 shape=None, case=None):
        import torch

        import decode_attention_gqa_amd as skv
        import synth
        self.torch, self.skv = torch, skv
        sh = shape or synth.Shape(1, 28, 4, 128, max_ctx)
        self.shape = sh
        self.L = layers
        self.S, self.blk = n_splits, block_len
        if case is None:
            log(f"[bench] generating layer data: max_ctx={max_ctx}")
            case = synth.make_offset_case(3, sh, max_ctx)
        self.case = case
        dev = torch.device("cuda", 0)
        k0 = torch.from_numpy(case.k).to(dev)
        v0 = torch.from_numpy(case.v).to(dev)
        q0 = torch.from_numpy(case.q).to(dev)
        # distinct allocations per layer: same values, different addresses
        self.k = [k0] + [k0.clone() for _ in range(layers - 1)]
        self.v = [v0] + [v0.clone() for _ in range(layers - 1)]
        self.q = [q0.clone() for _ in range(layers)]
        self.pos = torch.from_numpy(case.positions.copy()).to(dev)
        nb = skv.partials_bytes(sh.batch, sh.n_head, sh.head_dim, n_splits)
        self.part = [torch.empty(nb // 4, dtype=torch.float32, device=dev)
                     for _ in range(layers)]
        self.out = [torch.empty((sh.batch, sh.n_head, sh.head_dim),
                                dtype=torch.float32, device=dev)
                    for _ in range(layers)]
        self.scale = case.scale
        torch.cuda.synchronize()

    def step(self):
        for l in range(self.L):
            self.skv.decode_attn(self.q[l], self.k[l], self.v[l], self.pos,
                                 self.part[l], self.out[l], self.S, self.blk,
                                 self.scale)

    def partial(self, l):
        self.skv.partial(self.q[l], self.k[l], self.v[l], self.pos, self.part[l],
                         self.S, self.blk, self.scale)

    def combine(self, l):
        self.skv.combine(self.part[l], self.out[l], self.S)

    def capture(self):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        return g

    def set_nkv(self, nkv: int):
        self.pos.fill_(nkv - 1)
        self.torch.cuda.synchronize()


def time_replays(torch, graph, warmup: int, steps: int):
    """Per-replay milliseconds (events on the replay stream) and the total."""
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        graph.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total = evs[0].elapsed_time(evs[-1])
    return per, total, wall


def time_replays_cold(torch, graph, flush, warmup: int, steps: int):
    """Per-replay milliseconds with the Infinity Cache flushed before each
    replay: a 1 GiB read of other data runs on the same stream just before
    the first event, outside the timed window."""
    for _ in range(warmup):
        flush()
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush()
        a[i].record(stream)
        graph.replay()
        b[i].record(stream)
    torch.cuda.synchronize()
    return [a[i].elapsed_time(b[i]) for i in range(steps)]


def make_flush(torch, skv, gib: float = 1.0):
    n = int(gib * (1 << 30))
    buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    grid = torch.cuda.get_device_properties(0).multi_processor_count * 16
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    return lambda: skv.probe_read(buf, sink, grid)


def time_kernel(torch, launch, layers: int, reps: int):
    """Average duration of one launch of a kernel: `reps` launches rotating
    over the layers' buffers are captured into one hipGraph (so host launch
    cost is out of the picture) and the replays are timed with HIP events on
    the replay stream. Returns (mean, best) milliseconds per launch over 5
    replays. rocprofv3 --kernel-trace on --mode kernels times the same
    launches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for l in range(layers):
            launch(l)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            launch(i % layers)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / reps)
    del g
    return statistics.mean(per), min(per)


def hbm_read_probe(torch, skv, gib: float = 4.0, reps: int = 5) -> float:
    """Measured HBM read stream rate (GB/s) of a plain 16-byte load kernel."""
    n = int(gib * (1 << 30))
    buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cu * 16
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
    skv.probe_read(buf, sink, grid)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        skv.probe_read(buf, sink, grid)
        b.record()
        torch.cuda.synchronize()
        best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lay: Layers, nkv: int, budget_s: float = 12.0):
    """The fp64 oracle (one thread) on one layer at the same live length.
    Returns (the cpu_baseline record, the oracle's output of that layer)."""
    import numpy as np

    import oracle
    import synth
    c = lay.case
    pos = np.array([nkv - 1], np.int32)
    kv = synth.kv_bytes(lay.shape.n_kv_head, lay.shape.head_dim, nkv)
    runs, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.decode_attn(c.q, c.k, c.v, pos, lay.shape.n_kv_head,
                                 c.scale)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    model = cpu_model()
    return {"value": round(kv * runs / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle", "cpu_model": model,
            "cpus_visible": os.cpu_count(),
            "sample": f"{runs} x one layer (28q/4kv hd128, nkv {nkv}) in "
                      f"{el:.1f} s, single-threaded fp64 C on one core of "
                      f"{model} ({os.cpu_count()} cpus visible)"}, ref


def worst_errors(got, ref) -> dict:
    """Largest abs and rel error of a GPU output against the oracle's (rel
    over elements with |oracle| > 1e-6), and whether every element meets the
    bar |err| <= 5e-5 or |err| <= 1e-3 |oracle|."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    big = np.abs(ref) > 1e-6
    rel = np.where(big, err / np.where(big, np.abs(ref), 1.0), 0.0)
    ok = bool(np.all((err <= 5e-5) | (err <= 1e-3 * np.abs(ref))))
    return {"max_abs": float(err.max()), "max_rel": float(rel.max()),
            "within_bar": ok}


def load_traffic(nkv: int, n_splits: int, block_len: int):
    """HBM bytes per partial launch from the committed counter summary, if it
    was taken on the current kernel source and the same workload."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("partial_src_sha256_16") != source_hash():
        return None, "kernel changed since the counters were taken"
    if (t.get("nkv"), t.get("n_splits"), t.get("block_len")) != (nkv, n_splits,
                                                                 block_len):
        return None, "counters taken on another workload"
    return t.get("hbm_bytes_per_launch"), "rocprofv3 FETCH_SIZE+WRITE_SIZE"


# --------------------------------------------------------------------------
def run_main(args):
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    if not os.path.exists(skv.LIB_PATH):
        from decode_attention_gqa_amd import build as hip_build
        hip_build.build()
    props = torch.cuda.get_device_properties(0)
    cu = props.multi_processor_count
    max_ctx = synth.CFG3.max_ctx
    if args.n_splits:
        S, blk = args.n_splits, args.block_len
    else:
        S, blk = skv.pick_splits(1, 28, 4, 128, max_ctx, cu)
    lay = Layers(args.layers, max_ctx, S, blk)
    graph = lay.capture()

    points = []
    flush = None
    for nkv in sorted(set(args.points + [args.nkv])):
        lay.set_nkv(nkv)
        per, total, _ = time_replays(torch, graph, args.warmup, args.steps)
        med = statistics.median(per)
        kv = synth.kv_bytes(4, 128, nkv) * args.layers
        pt = {"nkv": nkv, "ms_per_step_median": round(med, 5),
              "us_per_layer": round(med * 1e3 / args.layers, 3),
              "kv_gbps": round(kv / (med * 1e-3) / 1e9, 1),
              "pct_hbm_peak": round(100 * kv / (med * 1e-3) / 1e9 /
                                    HBM_PEAK_GBPS, 2),
              "working_set_mb": round(kv / 1e6, 1)}
        if kv <= MALL_BYTES:
            # The whole step's K/V fits the Infinity Cache: the replays
            # above read it from there (warm). Cold: a 1 GiB read of other
            # data runs before each replay, outside the timed window.
            if flush is None:
                flush = make_flush(torch, skv)
            cold = statistics.median(time_replays_cold(
                torch, graph, flush, args.warmup, args.steps))
            pt.update({"resident": "Infinity Cache (warm)",
                       "us_per_layer_cold": round(cold * 1e3 / args.layers, 3),
                       "pct_hbm_peak_cold": round(
                           100 * kv / (cold * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)})
        else:
            pt["resident"] = "HBM"
        points.append(pt)
        log(f"[bench] nkv={nkv}: {points[-1]}")

    # headline: the timed K steps at --nkv
    lay.set_nkv(args.nkv)
    per, total, wall = time_replays(torch, graph, args.warmup, args.steps)
    ms_step = total / args.steps
    kv_layer = synth.kv_bytes(4, 128, args.nkv)
    value = kv_layer * args.layers / (ms_step * 1e-3) / 1e9

    # dominant kernel alone (partial), and the combine, events on its stream
    p_mean, p_med = time_kernel(torch, lay.partial, args.layers, args.kernel_reps)
    c_mean, c_med = time_kernel(torch, lay.combine, args.layers, args.kernel_reps)
    achieved = kv_layer / (p_mean * 1e-3) / 1e9
    traffic, traffic_src = load_traffic(args.nkv, S, blk)
    probe = hbm_read_probe(torch, skv) if not args.no_probe else None

    cpu, parity = None, None
    if not args.no_cpu:
        cpu, ref = cpu_baseline(lay, args.nkv, args.cpu_budget)
        # layer 0's output from the timed replays against the oracle's
        parity = worst_errors(lay.out[0].cpu().numpy(), ref)
        parity["sample"] = (f"layer 0 of the timed graph at nkv {args.nkv}, "
                            f"all 28 x 128 outputs")
    # every byte a layer moves: q, K+V, the records written by the partial
    # kernel and read back by the combine, and the output
    rec_bytes = skv.partials_bytes(1, 28, 128, S)
    total_layer = 28 * 128 * 4 + kv_layer + 2 * rec_bytes + 28 * 128 * 4
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"decode attention 28q/4kv hd128, nkv {args.nkv}, "
                               f"{args.layers} layers with separate KV buffers, "
                               f"hipGraph of partial+combine",
                   "nkv": args.nkv, "layers": args.layers, "max_ctx": max_ctx,
                   "n_splits": S, "block_len": blk, "kv_dtype": "fp16",
                   "q_dtype": "fp32", "out_dtype": "fp32",
                   "contraction": "fp16 matrix cores (v_mfma_f32_16x16x32_f16 "
                                  "for q.K, v_mfma_f32_16x16x16_f16 for p.V), "
                                  "fp32 accumulation; q and p as fp16 hi+lo "
                                  "pairs (about 22 significant bits)",
                   "global_batch": 1},
        "us_per_layer": round(ms_step * 1e3 / args.layers, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "partial_kernel<128,7>",
                     "bytes_per_launch": kv_layer,
                     "avg_launch_us": round(p_mean * 1e3, 3),
                     "best_batch_launch_us": round(p_med * 1e3, 3),
                     "traffic_source": traffic_src},
        "combine_avg_launch_us": round(c_mean * 1e3, 3),
        "hbm_read_probe_gbps": round(probe, 1) if probe else None,
        "pct_of_probe": round(100 * value / probe, 2) if probe else None,
        "total_bytes_per_layer": total_layer,
        "total_gbps": round(total_layer * args.layers / (ms_step * 1e-3) / 1e9, 1),
        "points": points,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "wall_s_timed": round(wall, 4),
        "device": props.name,
        "cu_count": cu,
    }
    print(json.dumps(line), flush=True)


def run_kernels(args):
    """Profiler workload: graphs of each layer's partial, combine and KV-cache
    append launches (HIP-event timed), then a plain copy of known size (the
    counter scale)."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    max_ctx = synth.CFG3.max_ctx
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if args.n_splits:
        S, blk = args.n_splits, args.block_len
    else:
        S, blk = skv.pick_splits(1, 28, 4, 128, max_ctx, cu)
    lay = Layers(args.layers, max_ctx, S, blk)
    lay.set_nkv(args.nkv)
    if args.per_head:   # the per-query-head form in place of the grouped one
        lay.partial = lambda l: skv.partial_per_head(
            lay.q[l], lay.k[l], lay.v[l], lay.pos, lay.part[l], S, blk,
            lay.scale)
    p_mean, _ = time_kernel(torch, lay.partial, args.layers, args.kernel_reps)
    c_mean, _ = time_kernel(torch, lay.combine, args.layers, args.kernel_reps)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    kn = torch.randn((1, 1, 4, 128), generator=gen, device="cuda")
    vn = torch.randn((1, 1, 4, 128), generator=gen, device="cuda")
    a_mean, _ = time_kernel(
        torch, lambda l: skv.append_kv(kn, vn, lay.k[l], lay.v[l], lay.pos),
        args.layers, args.kernel_reps)
    nbytes = args.copy_mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    skv.probe_copy(src, dst, cu * 16)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "kernels", "per_head": args.per_head,
                      "nkv": args.nkv, "n_splits": S,
                      "block_len": blk, "layers": args.layers,
                      "partial_launches": 6 * args.kernel_reps + args.layers,
                      "partial_avg_us_events": round(p_mean * 1e3, 3),
                      "combine_avg_us_events": round(c_mean * 1e3, 3),
                      "append_avg_us_events": round(a_mean * 1e3, 3),
                      "copy_bytes": nbytes,
                      "kv_bytes_per_partial": synth.kv_bytes(4, 128, args.nkv),
                      "partial_src_sha256_16": source_hash()}), flush=True)


def run_profile(args):
    """Profiler workload for one configuration (`--workload`): graphs of its
    partial-kernel launches and of its combine launches at the heuristic's
    split count over the layers' separate buffers (HIP-event timed), then a
    plain copy of known size (the counter scale). rocprofv3 --kernel-trace
    --stats and the FETCH_SIZE / WRITE_SIZE passes run on this mode; one JSON
    line carries what --summarize-pmc needs to turn counters into bytes."""
    import numpy as np
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    w = args.workload
    if w == "growing":
        sh, layers, nkv = synth.CFG3, args.layers, args.nkv
        case = synth.make_offset_case(3, sh, sh.max_ctx)
        case.positions[:] = nkv - 1
        name = f"28q/4kv hd128, nkv {nkv} (max_ctx {sh.max_ctx}), {layers} layers"
    elif w == "7b2k":
        sh, layers, nkv = synth.CFG2, synth.CFG2_LAYERS, synth.CFG2.max_ctx
        case = synth.make_case(2, sh, nkv)
        name = f"7B 28q/4kv hd128, nkv {nkv}, {layers} layers"
    elif w == "hd256":
        sh, layers, nkv = synth.CFG4, synth.CFG4_LAYERS, synth.CFG4_NKV
        case = synth.make_case(4, sh, nkv)
        name = f"16q/2kv hd256, nkv {nkv}, {layers} layers"
    elif w == "ragged":
        sh, layers = synth.CFG5, 1
        lengths = synth.cfg5_lengths()
        nkv = int(lengths.sum())
        # values do not affect timing: K/V drawn on the GPU below
        q = synth.make_q(5, 0, sh)
        case = synth.Case(sh, q, np.zeros((sh.batch, 1, sh.n_kv_head,
                                            sh.head_dim), np.float16),
                          None, (lengths - 1).astype(np.int32), sh.scale)
        name = (f"32 x 32q/8kv hd128, lengths U{{512..32768}} "
                f"(total {nkv} rows), 1 layer")
    else:
        raise SystemExit(f"unknown workload {w}")
    S, blk = skv.pick_splits(sh.batch, sh.n_head, sh.n_kv_head, sh.head_dim,
                             sh.max_ctx, cu)
    if w == "ragged":
        dev = torch.device("cuda", 0)
        g = torch.Generator(device=dev)
        g.manual_seed(5)

        class _L:
            pass
        lay = _L()
        lay.L = 1
        kk = torch.randn((sh.batch, sh.max_ctx, sh.n_kv_head, sh.head_dim),
                         generator=g, device=dev, dtype=torch.float16)
        vv = torch.randn(kk.shape, generator=g, device=dev,
                         dtype=torch.float16)
        qq = torch.from_numpy(case.q).to(dev)
        pos = torch.from_numpy(case.positions).to(dev)
        part = torch.empty(skv.partials_bytes(sh.batch, sh.n_head, sh.head_dim,
                                              S) // 4, device=dev)
        out = torch.empty((sh.batch, sh.n_head, sh.head_dim), device=dev)
        lay.partial = lambda l: skv.partial(qq, kk, vv, pos, part, S, blk,
                                            sh.scale)
        lay.combine = lambda l: skv.combine(part, out, S)
        kv = synth.kv_bytes(sh.n_kv_head, sh.head_dim, lengths)
    else:
        lay = Layers(layers, sh.max_ctx, S, blk, sh, case)
        kv = synth.kv_bytes(sh.n_kv_head, sh.head_dim, case.nkv)
    reps = args.kernel_reps
    p_mean, p_best = time_kernel(torch, lay.partial, lay.L, reps)
    c_mean, c_best = time_kernel(torch, lay.combine, lay.L, reps)
    nbytes = args.copy_mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    skv.probe_copy(src, dst, cu * 16)
    torch.cuda.synchronize()
    rec = skv.partials_bytes(sh.batch, sh.n_head, sh.head_dim, S)
    print(json.dumps({
        "mode": "profile", "workload": w, "description": name,
        "nkv": nkv, "n_splits": S, "block_len": blk, "layers": lay.L,
        # time_kernel: L eager launches, then a graph of `reps` launches
        # replayed 6 times
        "partial_launches": lay.L + 6 * reps,
        "combine_launches": lay.L + 6 * reps,
        "partial_avg_us_events": round(p_mean * 1e3, 3),
        "partial_best_us_events": round(p_best * 1e3, 3),
        "combine_avg_us_events": round(c_mean * 1e3, 3),
        "kv_bytes_per_partial": kv,
        "partial_gbps_events": round(kv / (p_mean * 1e-3) / 1e9, 1),
        "record_bytes": rec, "copy_bytes": nbytes,
        "partial_src_sha256_16": source_hash(),
        "combine_src_sha256_16": source_hash(COMBINE_SRCS)}), flush=True)


def run_ragged(args):
    """Ragged batch: 32 sequences, 32q/8kv hd128, nkv_b ~ U{512..32768}; one
    graph of partial + combine per (n_splits, block_len) point; prints one JSON
    line per point (KV GB/s over the live rows of all sequences)."""
    import numpy as np
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    sh = synth.CFG5
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    lengths = synth.cfg5_lengths()[:args.ragged_batch]
    if args.ragged_full:
        lengths[:] = sh.max_ctx
    sh = dataclasses.replace(sh, batch=len(lengths))
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    # K/V values do not affect timing: drawn on the GPU (seeded) for speed
    k = torch.randn((sh.batch, sh.max_ctx, sh.n_kv_head, sh.head_dim),
                    generator=g, device=dev, dtype=torch.float16)
    v = torch.randn(k.shape, generator=g, device=dev, dtype=torch.float16)
    q = torch.from_numpy(synth.make_q(5, 0, sh)).to(dev)
    pos = torch.from_numpy((lengths - 1).astype(np.int32)).to(dev)
    kv = synth.kv_bytes(sh.n_kv_head, sh.head_dim, lengths)
    out = torch.empty((sh.batch, sh.n_head, sh.head_dim), device=dev)
    S_h, blk_h = skv.pick_splits(sh.batch, sh.n_head, sh.n_kv_head, sh.head_dim,
                                 sh.max_ctx, cu)
    points = [(S_h, blk_h)] + [(s, 0) for s in args.sweep_splits] + \
             [(-(-sh.max_ctx // b), b) for b in args.sweep_blocks]
    for S, blk in points:
        part = torch.empty(skv.partials_bytes(sh.batch, sh.n_head, sh.head_dim, S)
                           // 4, device=dev)

        def step():
            skv.decode_attn(q, k, v, pos, part, out, S, blk, sh.scale)
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        per, total, _ = time_replays(torch, graph, args.warmup, args.steps)
        med = statistics.median(per)
        print(json.dumps({"ragged": not args.ragged_full, "batch": sh.batch,
                          "n_splits": S, "block_len": blk,
                          "heuristic": (S, blk) == (S_h, blk_h),
                          "kv_bytes": kv, "ms_per_step": round(med, 4),
                          "kv_gbps": round(kv / (med * 1e-3) / 1e9, 1)}),
              flush=True)
        del graph, part
        torch.cuda.empty_cache()


def run_configs(args):
    """The other decode workloads, one JSON line per (config, split) point:
    7B shape at 2K (28 layers, 117 MB: fits the 256 MB Infinity Cache) and
    the hd256 shape at 8,400 rows (12 layers, 206 MB) timed warm (cache-
    resident after earlier replays) and cold (cache flushed before each
    replay); the tiny case; the 32-sequence ragged batch at the heuristic."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    flush = make_flush(torch, skv)

    def emit(name, lay, S, blk, nkv_total):
        graph = lay.capture()
        kv = synth.kv_bytes(lay.shape.n_kv_head, lay.shape.head_dim,
                            nkv_total) * lay.L
        warm, _, _ = time_replays(torch, graph, args.warmup, args.steps)
        cold = time_replays_cold(torch, graph, flush, args.warmup, args.steps)
        del graph
        p_us = time_kernel(torch, lay.partial, lay.L, args.kernel_reps)[0] * 1e3
        c_us = time_kernel(torch, lay.combine, lay.L, args.kernel_reps)[0] * 1e3
        h = skv.pick_splits(*dataclasses.astuple(lay.shape), cu) == (S, blk)
        for label, per in (("warm", warm), ("cold", cold)):
            med = statistics.median(per)
            print(json.dumps({"config": name, "cache": label, "n_splits": S,
                              "block_len": blk, "heuristic": h,
                              "layers": lay.L,
                              "us_per_layer": round(med * 1e3 / lay.L, 3),
                              "kv_gbps": round(kv / (med * 1e-3) / 1e9, 1),
                              "partial_avg_us": round(p_us, 3),
                              "combine_avg_us": round(c_us, 3)}),
                  flush=True)

    sh = synth.CFG1
    case = synth.make_case(1, sh, sh.max_ctx)
    S, blk = skv.pick_splits(*dataclasses.astuple(sh), cu)
    # 64 layers of separate buffers, so that one replay outlasts the host's
    # submission of the next and the GPU time is what is measured
    for S_, blk_ in sorted({(S, blk), (synth.CFG1_SPLITS, 0)}):
        emit("tiny 4q/2kv hd64 nkv 256 x64 layers",
             Layers(64, sh.max_ctx, S_, blk_, sh, case), S_, blk_, sh.max_ctx)

    sh = synth.CFG2
    case = synth.make_case(2, sh, sh.max_ctx)
    S, blk = skv.pick_splits(*dataclasses.astuple(sh), cu)
    for S_ in sorted(set(synth.CFG2_SPLIT_SWEEP) | {S} | set(args.extra_splits)):
        lay = Layers(synth.CFG2_LAYERS, sh.max_ctx, S_, 0, sh, case)
        emit("7B 28q/4kv hd128 nkv 2048 x28 layers", lay, S_, 0, sh.max_ctx)
        del lay

    sh = synth.CFG4
    case = synth.make_case(4, sh, synth.CFG4_NKV)
    pts = {skv.pick_splits(*dataclasses.astuple(sh), cu)}
    pts |= {(-(-sh.max_ctx // b), b) for b in synth.CFG4_BLOCKS}
    pts |= {(s_, 0) for s_ in args.extra_splits}
    for S_, blk_ in sorted(pts):
        lay = Layers(synth.CFG4_LAYERS, sh.max_ctx, S_, blk_, sh, case)
        emit("hd256 16q/2kv nkv 8400 x12 layers", lay, S_, blk_, synth.CFG4_NKV)
        del lay
    torch.cuda.empty_cache()


def run_oracle(args):
    """The fp64 oracle (one thread) on each workload, median of 3 runs (one
    run for the 32-sequence batch), one JSON line per point. Needs no GPU."""
    import oracle
    import synth

    def timed(name, case, layers_note, reps=3):
        sh = case.shape
        runs = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.decode_attn(case.q, case.k, case.v, case.positions,
                               sh.n_kv_head, case.scale)
            runs.append(time.perf_counter() - t0)
        med = statistics.median(runs)
        kv = synth.kv_bytes(sh.n_kv_head, sh.head_dim, case.nkv)
        print(json.dumps({"config": name, "kind": "oracle", "cores": 1,
                          "ms_per_layer": round(med * 1e3, 2),
                          "kv_gbps": round(kv / med / 1e9, 4),
                          "note": layers_note}), flush=True)

    sh = synth.CFG1
    timed("tiny 4q/2kv hd64 nkv 256", synth.make_case(1, sh, sh.max_ctx), "1 layer")
    sh = synth.CFG2
    timed("7B 28q/4kv hd128 nkv 2048", synth.make_case(2, sh, sh.max_ctx),
          "1 layer (of 28)")
    sh = synth.CFG3
    for nkv in (2048, 16384, 32768):
        timed(f"7B 28q/4kv hd128 nkv {nkv}",
              synth.make_offset_case(3, sh, nkv), "1 layer (of 28)")
    sh = synth.CFG4
    timed("hd256 16q/2kv nkv 8400", synth.make_case(4, sh, synth.CFG4_NKV),
          "1 layer (of 12)")
    sh = synth.CFG5
    timed("ragged 32 x 32q/8kv hd128", synth.make_case(5, sh, synth.cfg5_lengths()),
          "1 layer step, all 32 sequences; one run (~50 s)", reps=1)


def run_step(args):
    """A whole decode step per layer: KV-cache append of the new row, then
    partial + combine, 28 layers in one graph, at several live lengths; the
    same step with the append folded into the partial kernel
    (splitkv_decode_step); plus the append kernel alone (graph of launches,
    HIP events)."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = synth.CFG3.max_ctx
    S, blk = skv.pick_splits(1, 28, 4, 128, max_ctx, cu)
    lay = Layers(args.layers, max_ctx, S, blk)
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    kn = [torch.randn((1, 1, 4, 128), generator=g, device=dev)
          for _ in range(lay.L)]
    vn = [torch.randn((1, 1, 4, 128), generator=g, device=dev)
          for _ in range(lay.L)]

    def append(l):
        skv.append_kv(kn[l], vn[l], lay.k[l], lay.v[l], lay.pos)

    def full():
        for l in range(lay.L):
            append(l)
            skv.decode_attn(lay.q[l], lay.k[l], lay.v[l], lay.pos, lay.part[l],
                            lay.out[l], S, blk, lay.scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        full()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        full()
    torch.cuda.synchronize()
    # the same step with the append folded into the partial kernel
    def folded():
        for l in range(lay.L):
            skv.decode_step(lay.q[l], kn[l], vn[l], lay.k[l], lay.v[l], lay.pos,
                            lay.part[l], lay.out[l], S, blk, lay.scale)

    with torch.cuda.stream(side):
        folded()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_f = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_f):
        folded()
    torch.cuda.synchronize()
    a_mean, _ = time_kernel(torch, append, lay.L, args.kernel_reps)
    row_bytes = 4 * 128 * (4 + 4 + 2 + 2)   # K,V fp32 read + fp16 written
    for nkv in args.points:
        lay.set_nkv(nkv)
        per, _, _ = time_replays(torch, graph, args.warmup, args.steps)
        med = statistics.median(per)
        per_f, _, _ = time_replays(torch, graph_f, args.warmup, args.steps)
        med_f = statistics.median(per_f)
        kv = synth.kv_bytes(4, 128, nkv) * lay.L
        print(json.dumps({"decode_step": True, "nkv": nkv, "n_splits": S,
                          "layers": lay.L,
                          "us_per_layer": round(med * 1e3 / lay.L, 3),
                          "kv_gbps": round(kv / (med * 1e-3) / 1e9, 1),
                          "folded_us_per_layer": round(med_f * 1e3 / lay.L, 3),
                          "folded_kv_gbps": round(kv / (med_f * 1e-3) / 1e9, 1),
                          "append_avg_us": round(a_mean * 1e3, 3),
                          "append_bytes": row_bytes}), flush=True)


def run_per_head(args):
    """A/B of the partial kernel's grid: grouped (one workgroup per split and
    KV head, all G query heads) against per-query-head (one workgroup per
    split and query head, every KV row read G times). 28 layers of partial +
    combine in one graph per variant and split count, plus the partial kernel
    alone."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = synth.CFG3.max_ctx
    S_g, _ = skv.pick_splits(1, 28, 4, 128, max_ctx, cu)
    variants = [("grouped", S_g)] + [("per_head", s) for s in args.sweep_splits]
    case = None
    for form, S in variants:
        lay = Layers(args.layers, max_ctx, S, 0, case=case)
        case = lay.case
        part_fn = skv.partial if form == "grouped" else skv.partial_per_head

        def step():
            for l in range(lay.L):
                part_fn(lay.q[l], lay.k[l], lay.v[l], lay.pos, lay.part[l], S, 0,
                        lay.scale)
                skv.combine(lay.part[l], lay.out[l], S)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for nkv in args.points:
            lay.set_nkv(nkv)
            per, _, _ = time_replays(torch, graph, args.warmup, args.steps)
            med = statistics.median(per)
            p_us = time_kernel(
                torch, lambda l: part_fn(lay.q[l], lay.k[l], lay.v[l], lay.pos,
                                         lay.part[l], S, 0, lay.scale),
                lay.L, args.kernel_reps)[0] * 1e3
            kv = synth.kv_bytes(4, 128, nkv)
            print(json.dumps({"form": form, "n_splits": S, "nkv": nkv,
                              "workgroups": S * (4 if form == "grouped" else 28),
                              "us_per_layer": round(med * 1e3 / lay.L, 3),
                              "partial_avg_us": round(p_us, 3),
                              "partial_kv_gbps": round(kv / (p_us * 1e-6) / 1e9,
                                                       1)}), flush=True)
        del graph, lay
        torch.cuda.empty_cache()


def run_long(args):
    """The headline shape past the 32K configs: 28q/4kv hd128 with max_ctx
    131,328, one graph of L layers x (partial + combine) replayed at live
    lengths 16K..128K (per-layer KV 32..256 MB, every layer in its own
    buffers), plus the partial kernel alone at each length."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = 131072 + 256
    S, blk = skv.pick_splits(1, 28, 4, 128, max_ctx, cu)
    lay = Layers(args.layers, max_ctx, S, blk)
    graph = lay.capture()
    for nkv in (16384, 32768, 65536, 131072):
        lay.set_nkv(nkv)
        per, _, _ = time_replays(torch, graph, args.warmup, args.steps)
        med = statistics.median(per)
        kv = synth.kv_bytes(4, 128, nkv)
        p_mean, _ = time_kernel(torch, lay.partial, lay.L, args.kernel_reps)
        print(json.dumps({"long": True, "nkv": nkv, "max_ctx": max_ctx,
                          "n_splits": S, "layers": lay.L,
                          "us_per_layer": round(med * 1e3 / lay.L, 3),
                          "kv_gbps": round(kv * lay.L / (med * 1e-3) / 1e9, 1),
                          "pct_hbm_peak": round(100 * kv * lay.L / (med * 1e-3)
                                                / 1e9 / HBM_PEAK_GBPS, 2),
                          "partial_avg_us": round(p_mean * 1e3, 3),
                          "partial_pct_hbm_peak": round(
                              100 * kv / (p_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}),
              flush=True)


def run_batch(args):
    """The headline shape with several sequences of one length: 28q/4kv
    hd128, max_ctx 33,024 (or --batch-max-ctx), batch 1..8, one graph of L
    layers x (partial + combine) per (batch, split count) replayed at
    --batch-lengths, every layer in its own buffers; the split counts are
    the heuristic's and the ones given by --extra-splits."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = args.batch_max_ctx or synth.CFG3.max_ctx
    for B in args.batches:
        sh = synth.Shape(B, 28, 4, 128, max_ctx)
        log(f"[bench] generating layer data: batch {B}, max_ctx={max_ctx}")
        case = synth.make_offset_case(3, sh, max_ctx)
        S_h, _ = skv.pick_splits(B, 28, 4, 128, max_ctx, cu)
        for S in [S_h] + [x for x in args.extra_splits if x != S_h]:
            lay = Layers(args.layers, max_ctx, S, 0, sh, case)
            graph = lay.capture()
            for nkv in [n for n in args.batch_lengths if n <= max_ctx]:
                lay.set_nkv(nkv)
                per, _, _ = time_replays(torch, graph, args.warmup, args.steps)
                med = statistics.median(per)
                kv = B * synth.kv_bytes(4, 128, nkv)
                p_mean, _ = time_kernel(torch, lay.partial, lay.L,
                                        args.kernel_reps)
                print(json.dumps({
                    "batch": B, "nkv": nkv, "max_ctx": max_ctx, "n_splits": S,
                    "heuristic": S == S_h, "layers": lay.L,
                    "us_per_layer": round(med * 1e3 / lay.L, 3),
                    "kv_gbps": round(kv * lay.L / (med * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * kv * lay.L / (med * 1e-3)
                                          / 1e9 / HBM_PEAK_GBPS, 2),
                    "partial_avg_us": round(p_mean * 1e3, 3),
                    "partial_pct_hbm_peak": round(
                        100 * kv / (p_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}),
                    flush=True)
            del graph, lay
            torch.cuda.synchronize()
            torch.cuda.empty_cache()


def run_rows(args):
    """Several query rows per sequence (speculative verification shape):
    28 layers of partial + combine in one graph, n_q rows per sequence at
    several live lengths, for the head layout given by --rows-heads (query
    heads, KV heads) and head size --rows-hd. The split count comes from
    the heuristic for several rows (splitkv_pick_splits_rows), plus those
    given by --extra-splits."""
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    max_ctx = synth.CFG3.max_ctx
    nh, nkvh = args.rows_heads
    hd = args.rows_hd
    sh = synth.Shape(1, nh, nkvh, hd, max_ctx)
    log(f"[bench] generating layer data: {nh}q/{nkvh}kv max_ctx={max_ctx}")
    base = Layers(args.layers, max_ctx, 1, 0, sh,
                  synth.make_case(3, sh, max_ctx))
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    for n_q in args.rows:
        S_h, blk = skv.pick_splits_rows(1, n_q, nh, nkvh, hd, max_ctx, cu)
        for S in [S_h] + [x for x in args.extra_splits if x != S_h]:
            qs = [torch.randn((1, n_q, nh, hd), generator=g, device=dev)
                  for _ in range(base.L)]
            parts = [torch.empty(skv.partials_bytes(1, n_q * nh, hd, S) // 4,
                                 device=dev) for _ in range(base.L)]
            outs = [torch.empty((1, n_q, nh, hd), device=dev)
                    for _ in range(base.L)]

            def step():
                for l in range(base.L):
                    skv.decode_attn_rows(qs[l], base.k[l], base.v[l], base.pos,
                                         parts[l], outs[l], S, blk, base.scale)

            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            for nkv in args.points:
                base.set_nkv(nkv)
                per, _, _ = time_replays(torch, graph, args.warmup, args.steps)
                med = statistics.median(per)
                kv = synth.kv_bytes(nkvh, hd, nkv) * base.L
                print(json.dumps({"heads": f"{nh}q/{nkvh}kv", "hd": hd, "rows": n_q,
                                  "n_splits": S, "heuristic": S == S_h, "nkv": nkv,
                                  "us_per_layer": round(med * 1e3 / base.L, 3),
                                  "us_per_row_layer": round(med * 1e3 / base.L / n_q, 3),
                                  "kv_gbps_once": round(kv / (med * 1e-3) / 1e9, 1)}),
                      flush=True)
            del graph, qs, parts, outs
            torch.cuda.empty_cache()


def run_sweep(args):
    import torch

    import decode_attention_gqa_amd as skv
    import synth
    max_ctx = synth.CFG3.max_ctx
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    case = None
    for S, blk in [(s, 0) for s in args.sweep_splits] + \
                  [(-(-max_ctx // b), b) for b in args.sweep_blocks]:
        lay = Layers(args.layers, max_ctx, S, blk, case=case)
        case = lay.case
        graph = lay.capture()
        for nkv in args.points:
            lay.set_nkv(nkv)
            per, total, _ = time_replays(torch, graph, args.warmup, args.steps)
            med = statistics.median(per)
            kv = synth.kv_bytes(4, 128, nkv) * args.layers
            print(json.dumps({"sweep": True, "n_splits": S, "block_len": blk,
                              "nkv": nkv, "cu": cu,
                              "us_per_layer": round(med * 1e3 / args.layers, 3),
                              "kv_gbps": round(kv / (med * 1e-3) / 1e9, 1)}),
                  flush=True)
        del lay, graph
        torch.cuda.empty_cache()


def summarize_pmc(fetch_dir: str, write_dir: str, copy_bytes: int,
                  kernels_json: str | None, out_path: str | None):
    """Per-dispatch HBM traffic of the partial kernel from two rocprofv3 --pmc
    runs of --mode kernels (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
    each scaled by what the same counter reads for the plain copy kernel of
    `copy_bytes` (which reads and writes exactly that many bytes)."""
    def means(directory, counter):
        vals = {}
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                              recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        vals.setdefault(r["Kernel_Name"], []).append(
                            float(r["Counter_Value"]))
        return {k: statistics.mean(v) for k, v in vals.items()}

    fetch = means(fetch_dir, "FETCH_SIZE")
    write = means(write_dir, "WRITE_SIZE")

    def pick(d, key):
        ks = [k for k in d if key in k]
        return d[ks[0]] if ks else None

    f_copy, w_copy = pick(fetch, "probe_copy_kernel"), pick(write, "probe_copy_kernel")
    f_part, w_part = pick(fetch, "partial_"), pick(write, "partial_")
    f_comb, w_comb = pick(fetch, "combine_kernel"), pick(write, "combine_kernel")
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    res = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "partial_fetch_bytes": round(f_part * 1024 * f_scale),
           "partial_write_bytes": round(w_part * 1024 * w_scale),
           "combine_fetch_bytes": round(f_comb * 1024 * f_scale),
           "combine_write_bytes": round(w_comb * 1024 * w_scale)}
    res["hbm_bytes_per_launch"] = res["partial_fetch_bytes"] + res["partial_write_bytes"]
    if kernels_json:
        with open(kernels_json) as f:
            meta = json.loads(f.read().strip().splitlines()[-1])
        for k in ("nkv", "n_splits", "block_len", "kv_bytes_per_partial",
                  "partial_src_sha256_16", "workload", "record_bytes",
                  "combine_src_sha256_16"):
            if k in meta:
                res[k] = meta[k]
        res["fetch_over_algorithmic"] = round(
            res["partial_fetch_bytes"] / meta["kv_bytes_per_partial"], 4)
        if "record_bytes" in meta:
            res["combine_fetch_over_records"] = round(
                res["combine_fetch_bytes"] / meta["record_bytes"], 4)
    print(json.dumps(res, indent=1))
    if out_path:
        with open(out_path, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")


def summarize_trace(trace_dir: str, layers: int, out_path: str | None):
    """Per-layer split of the layer graphs from a rocprofv3 --kernel-trace run
    of the default mode. The dispatches are sorted by start time; runs of
    alternating partial / combine dispatches are cut into replays of `layers`
    layers. Per layer: the partial kernel's duration, the gap to the
    combine's start, the combine's duration, the gap to the next layer's
    partial kernel, and the period from one partial start to the next
    (medians over all replays). The tracer stamps a dispatch that waits for
    the one before it as starting when that one ends, so the time between
    two kernels is counted in the second one's duration here."""
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"),
                          recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                kind = ("P" if "partial_" in name else
                        "C" if "combine_kernel" in name else "X")
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                             kind))
    rows.sort()
    runs, cur = [], []
    for st, en, kind in rows:
        expect = "P" if len(cur) % 2 == 0 else "C"
        if kind != expect:
            runs.append(cur)
            cur = []
            if kind != "P":
                continue
        cur.append((st, en, kind))
    runs.append(cur)
    n = 2 * layers
    replays = [r[i:i + n] for r in runs for i in range(0, len(r) - n + 1, n)]
    if not replays:
        raise SystemExit(f"no layer-graph replays found under {trace_dir}")
    pd, cd, gpc, gcp, per = [], [], [], [], []
    for r in replays:
        for i in range(0, n, 2):
            (ps, pe, _), (cs, ce, _) = r[i], r[i + 1]
            pd.append(pe - ps)
            cd.append(ce - cs)
            gpc.append(cs - pe)
            if i + 2 < n:
                gcp.append(r[i + 2][0] - ce)
                per.append(r[i + 2][0] - ps)

    def med(x):
        return round(statistics.median(x) / 1e3, 3)

    res = {"replays": len(replays), "layers": layers,
           "partial_us": med(pd), "gap_partial_to_combine_us": med(gpc),
           "combine_us": med(cd), "gap_combine_to_partial_us": med(gcp),
           "layer_period_us": med(per),
           "replay_us_per_layer": round(statistics.median(
               [(r[-1][1] - r[0][0]) / layers for r in replays]) / 1e3, 3)}
    print(json.dumps(res, indent=1))
    if out_path:
        with open(out_path, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--nkv", type=int, default=32768)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--points", type=int, nargs="*",
                    default=[2048, 4096, 8192, 16384, 32768])
    ap.add_argument("--n-splits", type=int, default=0)
    ap.add_argument("--block-len", type=int, default=0)
    ap.add_argument("--kernel-reps", type=int, default=56)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--sweep-splits", type=int, nargs="*",
                    default=[16, 32, 64, 128, 256, 512])
    ap.add_argument("--sweep-blocks", type=int, nargs="*", default=[128, 256, 512])
    ap.add_argument("--summarize-pmc", nargs=2, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", default=None, metavar="TRACE_DIR",
                    help="per-layer partial / gap / combine split of the layer "
                         "graphs in a rocprofv3 --kernel-trace run")
    ap.add_argument("--kernels-json", default=None)
    ap.add_argument("--write-traffic", default=None)
    ap.add_argument("--mode", choices=["main", "kernels", "ragged", "configs",
                                       "oracle", "step", "per_head", "rows",
                                       "long", "batch", "profile"],
                    default="main")
    ap.add_argument("--ragged-batch", type=int, default=32)
    ap.add_argument("--batches", type=int, nargs="*", default=[1, 2, 4, 8],
                    help="--mode batch: batch sizes")
    ap.add_argument("--batch-lengths", type=int, nargs="*",
                    default=[16384, 32768], help="--mode batch: live lengths")
    ap.add_argument("--batch-max-ctx", type=int, default=0,
                    help="--mode batch: cache rows per sequence (default 33,024)")
    ap.add_argument("--rows", type=int, nargs="*", default=[1, 2, 4, 8],
                    help="--mode rows: query rows per sequence to time")
    ap.add_argument("--rows-heads", type=int, nargs=2, default=[28, 4],
                    help="--mode rows: query heads and KV heads")
    ap.add_argument("--rows-hd", type=int, default=128,
                    help="--mode rows: head size")
    ap.add_argument("--per-head", action="store_true",
                    help="--mode kernels: time the per-query-head partial form")
    ap.add_argument("--extra-splits", type=int, nargs="*", default=[],
                    help="--mode configs: more split counts to time")
    ap.add_argument("--ragged-full", action="store_true",
                    help="every sequence at full length (uniform batch)")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--workload", default="growing",
                    choices=["growing", "7b2k", "hd256", "ragged"],
                    help="--mode profile: which configuration")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.layers, args.write_traffic)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                      args.copy_mib << 20, args.kernels_json, args.write_traffic)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU "
              "component (sharding by KV head or batch needs no exchange; see "
              "the design notes)", file=sys.stderr)
        return 2
    if args.sweep:
        run_sweep(args)
    elif args.mode == "profile":
        run_profile(args)
    elif args.mode == "kernels":
        run_kernels(args)
    elif args.mode == "ragged":
        run_ragged(args)
    elif args.mode == "configs":
        run_configs(args)
    elif args.mode == "oracle":
        run_oracle(args)
    elif args.mode == "step":
        run_step(args)
    elif args.mode == "per_head":
        run_per_head(args)
    elif args.mode == "rows":
        run_rows(args)
    elif args.mode == "long":
        run_long(args)
    elif args.mode == "batch":
        run_batch(args)
    else:
        run_main(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
