#!/usr/bin/env python3
"""Benchmark of one routed MoE layer on one MI355X.

A step is one moe_forward call -- routing plan, gather, grouped expert FFN and
combine -- over the prefill workload: T=2048 tokens, hidden 2560, 512 experts,
top-10, expert FFN 768, fp16 activations and weights, tm=16, seeded synthetic
routing (router logits N(0,1)). Inputs and weights are resident in HBM before
the timed region. Prints one JSON line.

The roofline object covers the dominant kernel (the gate/up + SwiGLU grouped
GEMM), bound by HBM: algorithmic bytes per launch (weights of the experts the
plan touches, gathered rows read, SwiGLU output written) divided by its
average launch time, measured with HIP events recorded by the library around
that kernel on its stream during the timed steps.

cpu_baseline: the CPU oracle (plain C, fp64, OpenMP over tokens) timed on the
host cores on a bounded sample of the same workload: the plan over all 2048
tokens plus gather and naive expert FFN for a prefix of the tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed (token,expert) rows/sec per MoE layer, T=2048 E=512 top-10; plan us/layer"
HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks (TFLOP/s) by element type; fp32 runs on the fp32 MFMA
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_RECORD = os.path.join(PROFILES, "prefill_fp16_hbm_traffic.md")
TIMER_EVERY = 5  # timed steps that also record the gate/up kernel's HIP events
GEMM_SOURCES = ["mixture_experts_routed_amd/csrc/ffn.hip", "mixture_experts_routed_amd/csrc/common.hpp",
                "mixture_experts_routed_amd/csrc/plan_wave.hpp"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "libbench_probe.so")


def build_probe() -> str:
    """Compile the benchmark's streaming-read probe (bench_probe.hip) for gfx950 into
    libbench_probe.so beside this file. It is a measurement helper of the benchmark,
    not part of the layer's library."""
    import subprocess

    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", PROBE_LIB + ".tmp", PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("bench probe build failed:\n" + r.stdout + r.stderr)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


_probe = None


def probe_lib():
    """The probe library (built by build_probe(); raises if missing)."""
    import ctypes

    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise FileNotFoundError(f"{PROBE_LIB} is missing: run bench.build_probe()")
        L = ctypes.CDLL(PROBE_LIB)
        L.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
        L.bench_stream_read.restype = ctypes.c_int
        _probe = L
    return _probe


def stream_read(src, sink, stream=None):
    """One streaming read of the GPU tensor `src` by the probe (on torch's current stream)."""
    import torch

    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = probe_lib().bench_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                       sink.data_ptr(), sink.numel(), s)
    if rc != 0:
        raise RuntimeError(f"bench_stream_read: status {rc}")


def probe_same_bytes(nbytes, dev, launches=8):
    """The read probe over nbytes (rounded up to 16) in one launch: median
    microseconds of single launches. Below 512 MiB each launch reads a region of
    a buffer at least 4x as large (and at least 1 GiB) that the launches before
    it did not read last, so that the Infinity Cache (256 MB) serves none of it;
    from 512 MiB on, every launch reads the same region (a sequential read of at
    least twice the cache's size gets no hits from it), which keeps the working
    set, and so the address-translation load, that of the kernel compared."""
    import torch

    nb = max(16, (int(nbytes) + 15) // 16 * 16)
    nreg = 1 if nb >= 512 << 20 else max(4 * nb, 1 << 30) // nb
    buf = torch.empty(nreg * nb, dtype=torch.uint8, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    ts = []
    for i in range(2 + launches):
        src = buf[(i % nreg) * nb: (i % nreg + 1) * nb]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        stream_read(src, sink)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(a.elapsed_time(b) * 1e3)
    del buf, sink
    us = float(np.median(ts))
    return {"bytes": nb, "us": round(us, 2), "gbs": round(nb / us / 1e3, 1)}


def gemm_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm_flags(name: str):
    """k_expert_gemm<T, GATEUP, GATHERED, PACKED>: the three flags from the (mangled
    or demangled) kernel name, or None"""
    import re
    m = re.search(r"k_expert_gemmI(?:DF16_|DF16b|f)Lb([01])ELb([01])ELb([01])E", name)
    if m:
        return tuple(g == "1" for g in m.groups())
    m = re.search(r"k_expert_gemm<[^,]+,\s*(true|false),\s*(true|false),\s*(true|false)", name)
    return tuple(g == "true" for g in m.groups()) if m else None


def gemm_is_gateup(name: str) -> bool:
    """GATEUP of a k_expert_gemm kernel name"""
    f = gemm_flags(name)
    return bool(f) and f[0]


def kernel_short_name(name: str) -> str:
    """a kernel's name in the traffic record: k_expert_gemm/gateup or /down (packed
    weights; _rowmajor with row-major ones), else the kernel's own name with its
    template arguments"""
    import re
    if "k_expert_gemm" in name:
        f = gemm_flags(name) or (False, False, True)
        return f"k_expert_gemm/{'gateup' if f[0] else 'down'}{'' if f[2] else '_rowmajor'}"
    m = re.search(r"moe::(k_\w+(?:<[^>]*>)?)|_ZN3moe(\d+)(k_\w+?)I", name)
    if m:
        return m.group(1) or m.group(3)
    return name[:40]


def pmc_summary(fetch_csv: str, write_csv: str, out_path: str, command: str) -> dict:
    """Per-kernel HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for a plain device copy of known size
    (the --copy-calibration-mib copy in the same run). Writes a markdown summary with a
    machine-readable record line and returns the record."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(dict)  # kernel -> dispatch -> KiB (summed over counter instances)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = vals[r["Kernel_Name"]]
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return vals

    short = kernel_short_name

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = None
    cf = [v for v in fetch.get(COPY_KERNEL, {}).values()]
    cw = [v for v in write.get(COPY_KERNEL, {}).values()]
    # the calibration copy is the large one; its size in KiB comes from WRITE_SIZE's own count
    copy_f, copy_w = max(cf), max(cw)
    mib = round(copy_w / 1024)
    copy_kib = mib * 1024
    kf, kw = copy_kib / copy_f, copy_kib / copy_w
    rows, rec = [], {"source_hash": gemm_source_hash(), "fetch_scale": kf, "write_scale": kw,
                     "copy_mib": mib, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if k == COPY_KERNEL or "elementwise" in k:
            continue
        f = list(fetch.get(k, {}).values())
        w = list(write.get(k, {}).values())
        fb = kf * sum(f) / max(len(f), 1) * 1024
        wb = kw * sum(w) / max(len(w), 1) * 1024
        rec["kernels"][short(k)] = {"read_bytes": fb, "write_bytes": wb, "dispatches": len(f)}
        rows.append((short(k), len(f), fb / 1e6, wb / 1e6))
    lines = [
        "# HBM traffic per dispatch: prefill_fp16 layer (T=2048, d=2560, E=512, top-10, f=768, fp16)",
        "",
        "Commands (from the repository root on one MI355X; each counter in its own run):",
        "",
        "```",
        command,
        "```",
        "",
        f"Calibration: a plain {mib} MiB device copy in the same runs read FETCH_SIZE = "
        f"{copy_f:.0f} KiB and WRITE_SIZE = {copy_w:.0f} KiB, so reads are scaled x{kf:.3f} "
        f"and writes x{kw:.3f}.",
        "",
        "| kernel | dispatches | read MB / dispatch | written MB / dispatch |",
        "|---|---:|---:|---:|",
    ] + [f"| `{k}` | {n} | {r:.2f} | {w:.2f} |" for k, n, r, w in rows] + [
        "",
        f"Kernel source hash (grouped GEMM sources at the time of the runs): {rec['source_hash']}",
        "",
        "traffic-record: " + json.dumps(rec),
        "",
    ]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    return rec


def recorded_traffic(kernel: str):
    """Calibrated HBM bytes per launch of `kernel` from the committed counter summary, or None
    when that summary was taken on different grouped-GEMM sources than the ones built now."""
    try:
        for line in open(TRAFFIC_RECORD):
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                if rec["source_hash"] != gemm_source_hash():
                    return None
                k = rec["kernels"][kernel]
                return k["read_bytes"] + k["write_bytes"]
    except (OSError, KeyError, ValueError):
        return None
    return None


def timed_us(fn, n):
    """mean microseconds per call of fn() over n back-to-back calls after 3 warm-up
    calls, from torch events on the current stream (the stream the library's calls
    are enqueued on)"""
    import torch

    for _ in range(3):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def queued_us(fn, n, dev):
    """mean microseconds per call of fn() over n back-to-back calls enqueued
    while the GPU is still busy with a 4 GiB fill, so that the calls run back
    to back on the GPU however long the host takes to issue each one (for
    launches shorter than the host's per-call cost); torch events on the
    current stream"""
    import torch

    for _ in range(3):
        fn()
    busy = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy.fill_(0)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    del busy
    return a.elapsed_time(b) * 1e3 / n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_fp16")
    ap.add_argument("--weights", choices=("packed", "rowmajor"), default="packed",
                    help="expert weights as moe_pack_weights lays them out (packed once before "
                         "the timed steps) or row-major as generated")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one captured step (a HIP graph of the step's layer "
                         "calls) instead of eager calls; stage times stay eager")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock target of the CPU oracle sample")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the calibrated HBM-traffic summary from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE run, WRITE_SIZE run) and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded in that summary")
    ap.add_argument("--host-weights", action="store_true",
                    help="time moe_forward_host_weights (expert weights in pinned host memory, "
                         "routed experts not yet in the device cache copied in per call) against "
                         "the device-weight layer on the same inputs, and exit")
    ap.add_argument("--host-slots", type=int, default=0,
                    help="expert slots of that device cache (0: the fewest one call needs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB (a "
                         "kernel of known traffic, to scale hardware byte counters)")
    return ap.parse_args()


def gateup_bytes(cfg, meta, T):
    """Algorithmic HBM bytes of one gate/up launch inside moe_forward: both weight
    matrices of every expert that has rows, each token's activation row read once
    (the kernel gathers its rows from x), the SwiGLU output written (nr rows)."""
    es = 2 if cfg.dtype != "f32" else 4
    nactive, nr = int(meta[4]), int(meta[2])
    return 2 * nactive * cfg.d * cfg.f * es + T * cfg.d * es + nr * cfg.f * es


def stage_flops(cfg, meta):
    """Algorithmic matrix FLOPs of the two grouped GEMMs of one moe_forward call, on the rows
    that hold an entry (tile padding not counted)."""
    nreal = int(meta[0]) - int(meta[6]) - int(meta[7])
    return {"gateup": 2 * nreal * cfg.d * 2 * cfg.f, "down": 2 * nreal * cfg.f * cfg.d}


def y_row_bytes(cfg):
    """bytes of one expert-output row as moe_forward keeps it: fp32 for fp32 layers;
    for fp16/bf16 the compact format (binary16 values and one exponent byte per
    128 columns)"""
    return cfg.d * 4 if cfg.dtype == "f32" else cfg.d * 2 + (cfg.d + 127) // 128


def stage_bytes(cfg, meta, T):
    """Algorithmic HBM bytes of each HBM-bound kernel of one moe_forward call."""
    es = 2 if cfg.dtype != "f32" else 4
    nactive, nr, nent = int(meta[4]), int(meta[2]), int(meta[0])
    nreal = nent - int(meta[6]) - int(meta[7])  # rows that hold an entry
    yb = y_row_bytes(cfg)
    return {
        "gateup": gateup_bytes(cfg, meta, T),
        # down: W_down of the active experts, h read, y written on real rows
        "down": nactive * cfg.f * cfg.d * es + nr * cfg.f * es + nreal * yb,
        # combine: y rows of every entry read, out written, pos read
        "combine": nreal * yb + T * cfg.d * 4 + nent * 4,
    }


def plan_bytes(cfg, meta):
    """Algorithmic bytes of the routing plan: ids read twice (histogram and placement),
    router weights read, pos written, stok and sw written on every row (pads included),
    the per-block offsets boff written, cnt and eoff written, one tile id per tm rows."""
    nent, nblk, nr, nt = int(meta[0]), int(meta[1]), int(meta[2]), int(meta[3])
    return 2 * nent * 4 + nent * 4 + nent * 4 + nr * 8 + nblk * cfg.E * 4 + 2 * cfg.E * 4 + nt * 4


def gather_bytes(cfg, meta, T):
    """Algorithmic bytes of the standalone gather: each token's row read once, every
    expert-sorted row written (pad rows as zeros)."""
    es = 2 if cfg.dtype != "f32" else 4
    return T * cfg.d * es + int(meta[2]) * cfg.d * es


def plan_gather_combine(cfg, meta, T, plan_us, gather_us, combine_us):
    """The plan, gather and combine together against the HBM peak (the layer's
    memory-bound steps other than the grouped GEMMs), with the 60% bar."""
    b = plan_bytes(cfg, meta) + gather_bytes(cfg, meta, T) + stage_bytes(cfg, meta, T)["combine"]
    us = plan_us + gather_us + combine_us
    gbs = b / (us * 1e3)
    # the same steps' bytes with fp32 expert outputs (the format the bar was set
    # for; 16-bit layers here read compact rows instead): the bar as a time
    nreal = int(meta[0]) - int(meta[6]) - int(meta[7])
    b32 = b - nreal * y_row_bytes(cfg) + nreal * cfg.d * 4
    time_bar = b32 / (0.6 * HBM_PEAK_GBS * 1e3)
    return {"bytes": b, "us": {"plan": round(plan_us, 2), "gather": round(gather_us, 2),
                               "combine": round(combine_us, 2), "total": round(us, 2)},
            "gbs": round(gbs, 1), "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 3),
            "bar": 0.6, "meets_bar": gbs / HBM_PEAK_GBS >= 0.6,
            "bytes_fp32_y": b32, "time_bar_us": round(time_bar, 1),
            "meets_time_bar": us <= time_bar,
            "note": "gather timed standalone (moe_gather on the same plan); moe_forward itself "
                    "fuses the gather into the gate/up operand loads, so its step has no gather "
                    "launch. time_bar_us: the time in which these steps would move their bytes "
                    "with fp32 expert outputs at 60% of the HBM peak; the compact outputs of "
                    "16-bit layers move fewer bytes in less time, which lowers frac"}


def cpu_baseline(cfg, ids, w, x, seconds):
    import oracle
    from mixture_experts_routed_amd import synth

    nth = oracle.nthreads_default()
    # weights on the host (regenerated from the same seeds)
    t0 = time.perf_counter()
    Wg, Wu, Wd = (synth.expert_weights(cfg, k) for k in ("gate", "up", "down"))
    log(f"cpu_baseline: host weights in {time.perf_counter() - t0:.1f}s, {nth} threads")

    def run(ntok):
        t = time.perf_counter()
        p = oracle.plan(ids, w, cfg.E, cfg.tm)
        sel = np.arange(ntok, dtype=np.int32)
        used = np.isin(p["stok"], sel)
        oracle.gather(x, np.where(used, p["stok"], -1).astype(np.int32))
        oracle.ffn(x, ids, w, Wg, Wu, Wd, cfg.dtype, True, tokens=sel, nthreads=nth)
        return time.perf_counter() - t

    probe = max(nth, 8)
    tp = run(probe)
    ntok = int(min(cfg.T, max(probe, round(probe * seconds / max(tp, 1e-3)))))
    ntok = max(nth, ntok // nth * nth)
    tt = run(ntok)
    rows = ntok * cfg.K
    return {"value": rows / tt, "unit": "rows/s", "cores": nth, "kind": "oracle",
            "sample": f"plan of all {cfg.T} tokens + gather + naive fp64 expert FFN of the first "
                      f"{ntok} tokens ({rows} routed rows), {tt:.1f} s wall"}


def host_weights_bench(args):
    """The layer with its expert weights in pinned host memory: rows/s of
    moe_forward_host_weights against the device-weight layer on the same inputs,
    cold (the cache cleared at the start of every step, so every routed expert is
    copied in at least once per step) and warm (one cache kept across steps), and
    the copy rate against a plain pinned-to-device copy of the same size. The
    bytes copied are counted from the cache's own record of each call, in an
    untimed replay of the same call sequence."""
    import torch

    from mixture_experts_routed_amd import abi, synth

    cfg = synth.CONFIGS[args.workload]
    T, K, E, d, f, tm = cfg.tokens_per_call, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm
    dt = abi.DTYPE_NAME[cfg.dtype]
    tdt = abi.TORCH_DTYPE[dt]
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
        return t.view(tdt) if a.dtype == np.uint16 else t

    wts = {k: up(synth.expert_weights(cfg, k)) for k in ("gate", "up", "down")}
    packed = args.weights == "packed"
    devw = abi.pack(wts["gate"], wts["up"], wts["down"]) if packed else dict(wts)
    torch.cuda.synchronize()
    hostw = {}
    for k, t in devw.items():  # pinned at allocation, then filled
        h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        h.copy_(t.cpu())
        hostw[k] = h
    xd, idsd, wd = up(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    chunks = [(xd[c * T:(c + 1) * T], idsd[c * T:(c + 1) * T], wd[c * T:(c + 1) * T])
              for c in range(cfg.ncalls)]
    ws = torch.empty(abi.moe_forward_workspace(T, K, E, d, f, tm, dt), dtype=torch.uint8,
                     device="cuda")
    slots = args.host_slots or min(E, T * K)  # the fewest slots one call needs
    cache = torch.empty(abi.moe_host_cache_bytes(T, K, E, d, f, dt, packed, slots),
                        dtype=torch.uint8, device="cuda")
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    per_expert = sum(t.numel() * t.element_size() for t in devw.values()) // E

    def init():
        abi.moe_host_cache_init(cache, E, d, f, dt, packed, slots)

    def calls(count=None):
        for cx, cids, cw in chunks:
            abi.moe_forward_host_weights(cx, cids, cw, hostw["gate"], hostw["up"], hostw["down"],
                                         packed, dt, T, K, E, d, f, tm, slots, cache, ws, out)
            if count is not None:
                count.append(int(cache[4:8].view(torch.int32).item()))

    def cold_step():
        init()
        calls()

    def dev_step():
        for cx, cids, cw in chunks:
            abi.forward(cx, cids, cw, wts["gate"], wts["up"], wts["down"], tm=tm, workspace=ws,
                        out=out, packed=devw if packed else None)

    n = max(1, args.steps)
    # experts copied per step: cold, one step from an empty cache; warm, the mean
    # over the n steps that follow timed_us's 3 warm-up steps from an empty cache
    # (the timed run below replays exactly that sequence of cache states)
    cold_n = []
    init()
    calls(cold_n)
    warm_n = []
    init()
    for _ in range(3):
        calls()
    for _ in range(n):
        calls(warm_n)
    cold_bytes = sum(cold_n) * per_expert
    warm_bytes = sum(warm_n) * per_expert / n
    cold_us = timed_us(cold_step, n)
    init()
    warm_us = timed_us(calls, n)
    dev_us = timed_us(dev_step, n)
    # the host link's plain rate: one pinned-to-device copy of one call's cold bytes
    nb = max(cold_bytes // cfg.ncalls, 1 << 20)
    src = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    copy_us = timed_us(lambda: dst.copy_(src, non_blocking=True), 5)
    copy_gbs = nb / copy_us / 1e3
    stage_us = cold_us - dev_us

    def rate(us):
        return T * K * cfg.ncalls / (us * 1e-6)

    line = {
        "metric": "routed_rows_per_s", "value": rate(cold_us),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": cold_us / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "weights": "host (pinned), " +
                   ("packed" if packed else "row-major"), "cache_slots": slots,
                   "cache": "cleared at the start of every step"},
        "host_weights": {
            "layer_us": round(cold_us, 1), "device_weight_layer_us": round(dev_us, 1),
            "copied_bytes_per_step": cold_bytes, "copied_experts_per_step": sum(cold_n),
            "stage_us": round(stage_us, 1),
            "stage_gbs": round(cold_bytes / stage_us / 1e3, 2) if stage_us > 0 else None,
            "plain_h2d_copy_gbs": round(copy_gbs, 2),
            "stage_frac_of_copy": round(cold_bytes / stage_us / 1e3 / copy_gbs, 3)
            if stage_us > 0 else None,
            "warm": {"layer_us": round(warm_us, 1), "rows_per_s": rate(warm_us),
                     "copied_bytes_per_step": round(warm_bytes),
                     "copied_experts_per_step": sum(warm_n) / n},
            "note": "stage_us = cold layer with host weights - layer with device weights, "
                    "same inputs; warm keeps the cache across steps, so the same inputs "
                    "every step copy in only what the previous steps evicted; the copy is "
                    "one pinned-to-device transfer of one call's cold bytes through the DMA "
                    "engines"},
    }
    print(json.dumps(line))


def main():
    args = parse()
    if args.host_weights:
        host_weights_bench(args)
        return
    if args.pmc_summary:
        rec = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], TRAFFIC_RECORD, args.pmc_command)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the layer is measured at one GPU's share; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_routed_amd import abi, synth

    cfg = synth.CONFIGS[args.workload]
    # a step is every layer call of the workload (one call, or one per token chunk)
    T, K, E, d, f, tm = cfg.tokens_per_call, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm
    ncalls = cfg.ncalls
    t0 = time.perf_counter()
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)
    tdt = abi.TORCH_DTYPE[abi.DTYPE_NAME[cfg.dtype]]

    def up(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        t = t.to("cuda")
        return t.view(tdt) if a.dtype == np.uint16 else t

    dev = torch.device("cuda:0")
    wts = {k: up(synth.expert_weights(cfg, k)) for k in ("gate", "up", "down")}
    packed, pack_ms = None, None
    if args.weights == "packed":
        # one-time layout change of the weights (model load), outside the steps
        torch.cuda.synchronize()
        tp = time.perf_counter()
        packed = abi.pack(wts["gate"], wts["up"], wts["down"])
        torch.cuda.synchronize()
        pack_ms = (time.perf_counter() - tp) * 1e3
    xd, idsd, wd = up(x), torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    chunks = [(xd[c * T:(c + 1) * T], idsd[c * T:(c + 1) * T], wd[c * T:(c + 1) * T])
              for c in range(ncalls)]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    ws = torch.empty(abi.moe_forward_workspace(T, K, E, d, f, tm, abi.DTYPE_NAME[cfg.dtype]),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    # timed steps record events around the gate/up kernel only, on every
    # TIMER_EVERY-th step (each event pair adds a few us of launch gap); every
    # stage is timed in a separate pass afterwards
    timer = abi.Timer(capacity=max(args.steps * ncalls, 1), stages=("gateup",))

    def step(tmr=None):
        for cx, cids, cw in chunks:
            abi.forward(cx, cids, cw, wts["gate"], wts["up"], wts["down"], tm=tm, workspace=ws,
                        out=out, timer=tmr, packed=packed)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    t1 = time.perf_counter()
    for i in range(args.steps):  # eager (also for the gate/up timer in graph mode)
        step(timer if i % TIMER_EVERY == 0 else None)
    torch.cuda.synchronize()
    if graph is None:
        wall = time.perf_counter() - t1
    ms = wall * 1e3 / args.steps
    st = timer.read()
    timer.close()
    breakdown = abi.Timer(capacity=max(args.steps * ncalls, 1))
    for _ in range(args.steps):
        step(breakdown)
    torch.cuda.synchronize()
    st_all = breakdown.read()
    breakdown.close()

    # per-step distribution (one event pair around each step, after the timed
    # steps): warm = back to back; cold = a 1 GiB buffer written before each step
    # evicts the 256 MB Infinity Cache and the L2s first
    ndist = max(1, min(args.steps, 30))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def distribution(cold: bool) -> dict:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(ndist)]
        for a, b in evs:
            if cold:
                flush.fill_(1)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        v = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        return {q: round(float(np.percentile(v, p)), 1) for q, p in (("p10", 10), ("p50", 50),
                                                                     ("p90", 90))}

    step_us = {"warm": distribution(False), "cold": distribution(True), "samples": ndist}

    # the benchmark's streaming-read probe over 2 GiB (16-byte non-temporal loads,
    # the weight streams' access pattern): the read rate this box attains
    del flush
    src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    for _ in range(2):
        stream_read(src, sink)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        stream_read(src, sink)
    c1.record()
    torch.cuda.synchronize()
    read_gbs = 10 * src.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, sink

    # the router step before the layer (moe_route_topk on the first call's logits),
    # timed on its own: it is not part of the layer step above
    logits = torch.from_numpy(synth.router_logits(cfg, T)).to(dev)
    r_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    r_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    for _ in range(3):
        abi.moe_route_topk(logits, T, E, K, r_ids, r_w)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        abi.moe_route_topk(logits, T, E, K, r_ids, r_w)
    ev1.record()
    torch.cuda.synchronize()
    route_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    L = abi.moe_forward_layout(T, K, E, d, f, tm, abi.DTYPE_NAME[cfg.dtype])
    meta = ws[L.meta: L.meta + 4 * abi.META_N].view(torch.int32).cpu().numpy()

    # the standalone gather (moe_gather) on the last call's plan, into the workspace's
    # xs rows (which moe_forward leaves unused when it fuses the gather)
    dt = abi.DTYPE_NAME[cfg.dtype]
    R = abi.moe_plan_sizes(T, K, E, tm).max_rows
    stok_d = ws[L.stok: L.stok + 4 * R].view(torch.int32)
    meta_d = ws[L.meta: L.meta + 4 * abi.META_N].view(torch.int32)
    xs_d = ws[L.xs: L.xs + R * d * tdt.itemsize]
    cx = chunks[-1][0]

    def gather():
        abi.moe_gather(cx, dt, T, d, stok_d, meta_d, R, xs_d)

    gather_us = timed_us(gather, args.steps)

    # the plan alone at the four sizes of the page's plan table (512 experts, top-10,
    # tm 16, this workload's routing): moe_plan into its own buffers
    plan_sizes = {}
    if (E, K, tm) == (512, 10, 16):
        for Tp in (128, 512, 1024, 2048):
            pid, pw = synth.routing(cfg, Tp)
            pid, pw = torch.from_numpy(pid).to(dev), torch.from_numpy(pw).to(dev)
            o = abi.plan(pid, pw, E, tm)  # allocates the outputs once

            def plan_call():
                abi.moe_plan(pid, pw, Tp, K, E, tm, o["cnt"], o["eoff"], o["tiles"], o["stok"],
                             o["sw"], o["pos"], o["boff"], o["meta"], o["scratch"])

            us_p = queued_us(plan_call, 40, dev)
            plan_sizes[str(Tp)] = {"us": round(us_p, 2),
                                   "padded_rows": int(o["meta"][2].item()),
                                   "nblk": int(o["meta"][1].item())}

    # the same steps with row-major weights (moe_forward, the contract's call)
    rowmajor = None
    if packed is not None:
        def step_rm():
            for cx_, cids, cw in chunks:
                abi.forward(cx_, cids, cw, wts["gate"], wts["up"], wts["down"], tm=tm,
                            workspace=ws, out=out)

        for _ in range(args.warmup):
            step_rm()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            step_rm()
        torch.cuda.synchronize()
        ms_rm = (time.perf_counter() - t2) * 1e3 / args.steps
        rowmajor = {"value": cfg.T * K / (ms_rm * 1e-3), "unit": "rows/s",
                    "ms_per_step": ms_rm,
                    "note": "moe_forward with the row-major weights, same inputs and steps"}
    us = {k: 1e3 * v[0] / max(v[1], 1) for k, v in st_all.items()}
    # a call of at most 64 entries (one work item per expert) is planned inside
    # moe_forward's gate/up launch: no plan launch to time there, so the plan
    # is timed as moe_plan alone (its one-wavefront launch) on the last call
    plan_in_gateup = all(st_all[k][1] == 0 for k in ("hist", "scan", "place"))
    plan_us = us["hist"] + us["scan"] + us["place"]
    if plan_in_gateup:
        ids_last, w_last = chunks[-1][1], chunks[-1][2]
        o_pl = abi.plan(ids_last, w_last, E, tm)

        def plan_alone():
            abi.moe_plan(ids_last, w_last, T, K, E, tm, o_pl["cnt"], o_pl["eoff"], o_pl["tiles"],
                         o_pl["stok"], o_pl["sw"], o_pl["pos"], o_pl["boff"], o_pl["meta"],
                         o_pl["scratch"])

        plan_us = queued_us(plan_alone, 40, dev)
    gu_us = 1e3 * st["gateup"][0] / max(st["gateup"][1], 1)  # from the timed steps
    gu_bytes = gateup_bytes(cfg, meta, T)
    gu_s = gu_us * 1e-6
    achieved = gu_bytes / gu_s / 1e9
    same_bytes = probe_same_bytes(gu_bytes, dev)
    flops = stage_flops(cfg, meta)
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    # the gate/up launch is bound by the matrix cores when its arithmetic intensity
    # (algorithmic FLOPs per algorithmic byte) is above the ridge peak FLOP/s / HBM B/s
    mfma_bound = flops["gateup"] / gu_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"kernel": "gateup_swiglu", "bound": "mfma",
                "achieved": flops["gateup"] / gu_s / 1e12, "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": flops["gateup"] / gu_s / 1e12 / mfma_peak, "traffic": None,
                "hbm_gbs": round(achieved, 1),
                "algorithmic_flops_per_launch": flops["gateup"],
                "algorithmic_bytes_per_launch": gu_bytes}
    else:
        roof = {"kernel": "gateup_swiglu", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                # the committed counter record covers the prefill workload only
                "traffic": recorded_traffic("k_expert_gemm/gateup" +
                                            ("" if packed is not None else "_rowmajor"))
                           if cfg.name == "prefill_fp16" else None,
                "algorithmic_bytes_per_launch": gu_bytes}
    roof["read_probe_same_bytes"] = dict(
        same_bytes, launch_frac=round(achieved / same_bytes["gbs"], 3),
        note="the read probe reading the gate/up launch's algorithmic byte count in one launch "
             "(a fresh region of a larger buffer each time, so nothing comes from the Infinity "
             "Cache), median of single launches timed by events; launch_frac = the gate/up "
             "launch's algorithmic GB/s over the probe's: a plain read of the same bytes in one "
             "launch, ramp-up and drain included, reaches this rate")
    rows = cfg.T * K
    res = {
        "metric": METRIC, "value": rows / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": d, "E": E, "top_k": K, "f": f, "tm": tm,
                   "layer_calls_per_step": ncalls,
                   "launch": "one HIP graph replay per step" if graph is not None
                             else "eager kernel launches",
                   "routing": {"none": "router logits N(0,1)", "normal0.5": "router logits N(0,1) "
                               "+ per-expert N(0,0.5) bias", "zipf1.1": "router logits N(0,1) + "
                               "Zipf(1.1)-ranked per-expert bias"}[cfg.bias] +
                              ", softmax top-k renormalised" +
                              (", tail-skipped slots (weight < %.2f/K) routed nowhere" % cfg.tail_skip
                               if cfg.tail_skip else ""),
                   "weights": ("packed once into the MFMA tile layout by moe_pack_weights before "
                               "the timed steps (%.1f ms)" % pack_ms) if packed is not None
                              else "row-major [E][d][f] / [E][f][d] as generated"},
        "plan_us": plan_us,
        "plan_note": ("moe_forward plans this call inside its gate/up launch (at most 64 "
                      "entries, one work item per expert); plan_us is moe_plan alone on the "
                      "last call's routing (its one-wavefront launch), 40 calls queued back to "
                      "back behind a 4 GiB fill, by events") if plan_in_gateup else
                     "the plan's launches in moe_forward, per-kernel HIP events",
        "route_us": route_us,
        "stages_us": {k: round(v, 2) for k, v in us.items() if st_all[k][1] > 0},
        "stages_note": "per-kernel HIP events in a pass after the timed steps (events around "
                       "every kernel); the timed steps record the gate/up kernel only, on every "
                       f"{TIMER_EVERY}th step",
        "step_us_note": "one event pair per step, after the timed steps; cold: a 1 GiB buffer "
                        "is written before each step",
        "stages_gbs": {k: round(b / (us[k] * 1e3), 1) for k, b in stage_bytes(cfg, meta, T).items()
                       if us.get(k)},
        "gather_us": round(gather_us, 2),
        "plan_gather_combine": plan_gather_combine(
            cfg, meta, T, plan_us, gather_us, us["combine"]),
        "plan_us_by_T": plan_sizes or None,
        "plan_us_by_T_note": "moe_plan alone (one launch up to 32,768 entries), 512 experts, "
                             "top-10, tm 16, at the token counts of the page's plan table, 40 "
                             "calls queued back to back behind a 4 GiB fill, by events; "
                             "padded_rows is the plan's nr",
        "rowmajor": rowmajor,
        "step_us": step_us,
        "plan_meta": {n: int(v) for n, v in zip(abi.META_FIELDS, meta)},
        "stages_tflops": {k: round(v / (us[k] * 1e6), 1) for k, v in flops.items() if us.get(k)},
        "roofline": dict(roof, read_probe_gbs=round(read_gbs, 1),
                         read_probe_note="same run: the benchmark read probe (bench_probe.hip) over 2 GiB (each workgroup "
                                         "one contiguous chunk, 16-byte non-temporal loads, "
                                         "no compute) reaches this rate"),
    }
    if args.workload != "prefill_fp16":
        # the headline metric is quoted on the prefill layer; other workloads report
        # their own throughput under a metric name of their own
        res["metric"] = f"routed (token,expert) rows/sec, {cfg.name}"
        res["roofline"]["note"] = ("algorithmic %s of the last call's gate/up launch over the "
                                   "mean gate/up launch time"
                                   % ("FLOPs (rows holding an entry)" if mfma_bound else "bytes"))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, ids[:T], w[:T], x[:T], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
