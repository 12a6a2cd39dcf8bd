#!/usr/bin/env python3
"""Throughput of the MXFP8 quantizer on one MI355X.

One step = one pass of the hot path over one [16384, 7168] bf16 activation
batch (0.5 * Student-t(3), seeded): MXFP8 column-wise (groups of 32 tokens),
row-wise (groups of 32 along hidden) and the fused row-wise fake-quant, all
from a single read of the input.  ``value`` is algorithmic bytes (bf16 in +
codes, scales and fake-quant out) per second over the timed steps, inputs
resident in HBM.  Prints one JSON line.

Steps cycle through BATCHES resident batches, each with its own outputs
(distinct HBM addresses, 2.8 GB in all), so no step finds its input in the
256 MB Infinity Cache that the previous step just streamed through: the
timed rate is an HBM rate.  The act_16384 breakdown workloads use the same
batches; every other workload is timed over enough copies of its inputs that
at least 1 GB of other inputs is read between two reads of the same one (a
kernel whose input is small, such as a dequantization, gets more copies), and
the codes a dequantizer reads are written into every copy before timing.
Every timed workload, the streams included, follows an untimed warm-up of at
least 20 ms (warm_up); the main step follows the streams and its own warm-up
steps.  Timed right after host-side set-up, the GPU runs slower for a few
milliseconds: 5-7% on a 50 us kernel after 16 launches, 1% on the main step.

Besides the timed steps it reports, in the same line:
  roofline      the one-pass kernel's achieved GB/s (HIP events on the stream
                it runs on) against MI355X's 8 TB/s HBM peak and against the
                streaming ceiling of its own read:write mix, plus HBM traffic
                from the committed rocprofv3 counter summary when it still
                matches the kernel source
  ceilings      per read:write mix (read, write, copy, row-wise quantize,
                one-pass, dequantize, FP4 encode, FP4 dequantize, FP8 block to
                MXFP8), the best rate of several trivial-arithmetic streaming
                patterns (bench_streams.hip: the quantizers' 512-column tiles
                and half-width 256-column ones, in the plain and the XCD
                row-block order, and grid-stride walks) over cold inputs;
                ceiling_runs lists every pattern's rate
  cpu_baseline  the CPU oracle (single-threaded C) timed on a bounded sample
                of the same workload, and the same sharded over host threads
  breakdown     every other quantizer workload (row-wise weight, grouped MoE
                experts, block-FP8, NVFP4, dequantizers), each timed on its own;
                the quantizers and dequantizers also as a fraction of their
                mix's ceiling (measured on the [16384, 7168] batches); the
                [8192, 8192] kernels also against the streams measured on
                their own buffers (ceilings_square_8192), NVFP4 quantize
                against its read-only and FP4-encode streams back to back
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
BATCHES = 4            # resident batches the main step loop cycles through
COLD_INPUT_BYTES = 1e9  # other workloads: input bytes read between two reads of one copy
MAX_COPIES = 32
QT_PAD = 256  # bytes between the transposed codes' rows beyond `rows`, for the padded entry
METRIC = "MXFP8 quantize GB/s (bf16 in + fp8/scale out) and % of HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "block_scaled_precision_mxfp8_amd", "csrc", f)
                  for f in ("mx_kernels.hip", "mxq_device.hpp")]


STREAMS_SRC = os.path.join(ROOT, "bench_streams.hip")
STREAMS_LIB = os.path.join(ROOT, "libbench_streams.so")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def streams_hash() -> str:
    """Hash of the streaming-ceiling kernels' sources and flags."""
    from block_scaled_precision_mxfp8_amd import build as pb
    h = hashlib.sha256(" ".join(pb.HIPFLAGS).encode())
    for p in (STREAMS_SRC, os.path.join(pb.CSRC, "mxq_device.hpp")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build_streams() -> str:
    """Compile bench_streams.hip (the streaming-ceiling kernels) for gfx950."""
    import subprocess
    from block_scaled_precision_mxfp8_amd import build as pb
    tmp = STREAMS_LIB + ".tmp"
    subprocess.run([pb.HIPCC, *pb.HIPFLAGS, "-shared", f"-DSTREAMS_BUILD_ID=\"{streams_hash()}\"",
                    "-I", pb.CSRC, STREAMS_SRC, "-o", tmp], check=True)
    os.replace(tmp, STREAMS_LIB)
    return STREAMS_LIB


def load_streams():
    """The streaming-ceiling library (built first if missing; a build from
    other sources is refused)."""
    if not os.path.exists(STREAMS_LIB):
        build_streams()
    L = ctypes.CDLL(STREAMS_LIB)
    L.bench_streams_build_id.restype = ctypes.c_char_p
    if L.bench_streams_build_id().decode() != streams_hash():
        raise RuntimeError(f"{STREAMS_LIB} was built from other sources: run "
                           f"__graft_entry__.build()")
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.bench_stream_tiled.restype = ctypes.c_int
    L.bench_stream_tiled.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.bench_stream_flat.restype = ctypes.c_int
    L.bench_stream_flat.argtypes = [ctypes.c_int, vp, i64, vp, vp, vp, vp, ctypes.c_int, vp]
    L.bench_streams_kinds.restype = ctypes.c_int
    return L


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so a comment edit does not invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = kernel_source_hash()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 3 and parts[0] == "traffic" and parts[1] == workload:
                kv = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
                if kv.get("source") != src:
                    return None
                return float(kv["bytes"])
    return None


# Streaming-ceiling mixes in bench_streams.hip's kind order, and the bytes each
# moves per element (tiled patterns, which carry the scale stream; flat ones).
MIXES = ["read", "write", "copy", "row", "onepass", "dequant", "fp4", "fp4dq", "requant"]
MIX_BYTES = {
    "read": (2.0, 2.0), "write": (2.0, 2.0), "copy": (4.0, 4.0),
    "row": (3.0 + 1 / 32, 3.0), "onepass": (6.0 + 1 / 32, 6.0),
    "dequant": (3.0 + 1 / 32, 3.0), "fp4": (2.5 + 1 / 32, 2.5), "fp4dq": (2.5 + 1 / 32, 2.5),
    "requant": (2.0 + 1 / 32, 2.0)}
MIX_DESC = {
    "read": "2 B read per element", "write": "2 B written", "copy": "2 B read : 2 written",
    "row": "2 B read : 1 + 1/32 written", "onepass": "2 B read : 4 + 1/16 written",
    "dequant": "1 + 1/32 B read : 2 written", "fp4": "2 B read : 1/2 + 1/32 written",
    "fp4dq": "1/2 + 1/32 B read : 2 written", "requant": "1 B read : 1 + 1/32 written"}


WARM_S = 0.02  # untimed warm-up before each timed workload, at least this long


def warm_up(launch, arg_sets, min_launches=16):
    """Untimed launches cycling over arg_sets, in rounds of max(min_launches,
    len(arg_sets)) ended by a synchronize, until WARM_S has passed.  After a
    pause in GPU work (host-side set-up between workloads) the part takes a
    few milliseconds to come back to full speed: a 50 us kernel timed after
    16 launches read 5-7% slower than after 10 ms of launches."""
    import torch
    n = max(min_launches, len(arg_sets))
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(n):
            launch(arg_sets[i % len(arg_sets)])
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARM_S:
            return


def measure_ceilings(L, batches, rows, cols, stream, sp, iters=20, mixes=None):
    """Best GB/s per mix over the tiled (512- or 256-column tiles; R = 1, 2,
    4, 8 rows per wave; plain or XCD row-block order; up to 8 or at most 5
    resident workgroups per CU) and flat
    (U = 2, 4, 8 vectors in flight; 1024, 2048, 4096 workgroups) patterns,
    each timed like the quantizers: back-to-back launches cycling over cold
    inputs after an untimed warm-up.  The mixes that read x cycle over the
    batches, as the bench step does.  The three that read codes (1 B or 1/2 B per
    element) would find 4 batches' codes in the 256 MB Infinity Cache, so they
    cycle over every code region the batches hold (8 for 1-byte codes, 16 for
    half-byte ones): 0.85-0.93 GB of other codes pass between two reads of one."""
    import torch
    assert L.bench_streams_kinds() == len(MIXES)
    e = rows * cols
    sink = torch.empty((16,), dtype=torch.int32, device=batches[0]["x"].device)

    def A(t, off=0):
        return ctypes.c_void_p(t.data_ptr() + off)

    # per mix: the argument sets (x, codes, o8b, o16, row scales) it cycles over
    plain = [(A(d["x"]), A(d["qc"]), A(d["qr"]), A(d["fq"]), A(d["sr"])) for d in batches]
    codes1 = [(A(d["x"]), A(d[k]), A(d["qr"]), A(d["fq"]), A(d["sr"]))
              for k in ("qc", "qr") for d in batches]
    codes_half = [(A(d["x"]), A(d[k], h * (e // 2)), A(d["qr"]), A(d["fq"]), A(d["sr"]))
                  for k in ("qc", "qr") for h in (0, 1) for d in batches]
    # FP8 block -> MXFP8 writes codes too: to the fake-quant buffer, not the codes it reads
    codes_rq = [(A(d["x"]), A(d[k]), A(d["fq"]), A(d["fq"]), A(d["sr"]))
                for k in ("qc", "qr") for d in batches]
    sources = {m: plain for m in MIXES}
    sources["dequant"], sources["fp4dq"], sources["requant"] = codes1, codes_half, codes_rq

    def timed(launch, srcs):
        warm_up(launch, srcs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            launch(srcs[i % len(srcs)])
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / iters * 1e-3

    runs = {}
    for v in range(32 * len(MIXES)):
        mix, R = MIXES[(v // 4) % len(MIXES)], 1 << (v % 4)
        order = " xcd" if (v // (4 * len(MIXES))) % 2 else ""
        order += " 256c" if (v // (8 * len(MIXES))) % 2 else ""
        order += " cap5" if v >= 16 * len(MIXES) else ""
        if mixes is not None and mix not in mixes:
            continue

        def go(a, v=v):
            st = L.bench_stream_tiled(v, a[0], rows, cols, a[1], a[2], a[3], a[4], A(sink), sp)
            if st != 0:
                raise RuntimeError(f"bench_stream_tiled({v}) status {st}")
        runs[f"{mix} tiled R{R}{order}"] = (mix, MIX_BYTES[mix][0] * e / timed(go, sources[mix]) / 1e9)
    for v in range(3 * len(MIXES)):
        mix, U = MIXES[v // 3], (2, 4, 8)[v % 3]
        if mixes is not None and mix not in mixes:
            continue
        for grid in (1024, 2048, 4096):
            def go(a, v=v, grid=grid):
                st = L.bench_stream_flat(v, a[0], e // 8, a[1], a[2], a[3], A(sink), grid, sp)
                if st != 0:
                    raise RuntimeError(f"bench_stream_flat({v}) status {st}")
            runs[f"{mix} flat U{U} grid{grid}"] = (
                mix, MIX_BYTES[mix][1] * e / timed(go, sources[mix]) / 1e9)
    best = {}
    for name, (mix, gbs) in runs.items():
        if mix not in best or gbs > best[mix]["GB/s"]:
            best[mix] = {"GB/s": round(gbs, 1), "pattern": name, "bytes": MIX_DESC[mix]}
    return best, {k: round(g, 1) for k, (_, g) in runs.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-breakdown", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of the activation the CPU oracle baseline processes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world} "
              f"requested): the quantizers run per GPU shard with no exchange except NVFP4's "
              f"4-byte global-amax MAX, which this single-GPU build does not implement; "
              f"run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_precision_mxfp8_amd as mxq
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    lib = mxq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr())

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {mxq.status_string(st)}")

    # ------------------------------------------------------------------
    # main workload: one-pass column-wise + row-wise + fake-quant
    # ------------------------------------------------------------------
    rows, cols = workloads.SHAPES["act_16384"]
    log(f"generating act_16384 [{rows}, {cols}]")
    xb = workloads.act_16384()
    x0 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    e = rows * cols

    def batch(src):
        return {"x": src.clone(),
                "qc": torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                "sc": torch.empty(((rows + 31) // 32, cols), dtype=torch.uint8, device=dev),
                "qr": torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                "sr": torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev),
                "fq": torch.empty((rows, cols), dtype=torch.bfloat16, device=dev),
                # room for qT rows padded by QT_PAD bytes (the padded entry)
                "qt": torch.empty((cols * (rows + QT_PAD),), dtype=torch.uint8, device=dev),
                "st": torch.empty((cols, (rows + 31) // 32), dtype=torch.uint8, device=dev),
                "S1": torch.empty((rows, cols // 128), dtype=torch.float32, device=dev),
                "q4": torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                "s4": torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)}

    batches = [batch(x0) for _ in range(BATCHES)]
    del x0
    step_bytes = 2 * e + e + e // 32 + e + batches[0]["sc"].numel() + 2 * e

    def launch_fused(d):
        check(lib.mxq_quantize_colwise(P(d["x"]), rows, cols, P(d["qc"]), P(d["sc"]), P(d["qr"]),
                                       P(d["sr"]), P(d["fq"]), sp), "mxq_quantize_colwise")

    # Streaming ceilings: per read:write mix, the best of several access
    # patterns with trivial arithmetic (bench_streams.hip), over the same cold
    # batches.  The quantizer kernels are reported against the ceiling of
    # their own mix as well as against the 8 TB/s peak.  Measured before the
    # main step, so that the step is not timed while the GPU is still coming
    # back from the host-side set-up above (about 1% on the step).
    ceilings, ceiling_runs = measure_ceilings(load_streams(), batches, rows, cols, stream, sp)

    log(f"warmup {args.warmup}")
    for i in range(max(args.warmup, BATCHES)):
        launch_fused(batches[i % BATCHES])
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch_fused(batches[i % BATCHES])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # The step is exactly one launch of the one-pass kernel on `stream`, so the
    # HIP-event average over the timed region is the kernel's average launch
    # duration.  Per-launch spread: events recorded between back-to-back
    # launches (each interval also holds one event's own overhead).
    kern_ms = ms_per_step
    nl = max(10, min(args.steps, 50))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(nl):
        launch_fused(batches[i % BATCHES])
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    durs = [evs[i].elapsed_time(evs[i + 1]) for i in range(nl)]
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic("act_16384")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "mx_colwise_kernel<true,true,true,false,8>", "algorithmic_bytes": step_bytes,
                "avg_launch_us": round(kern_ms * 1e3, 2),
                "per_launch_us_min_max": [round(min(durs) * 1e3, 2), round(max(durs) * 1e3, 2)]}
    log(f"main: {value:.1f} GB/s per step, kernel {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBS:.1%})")

    oc = ceilings["onepass"]
    roofline["ceiling"] = {"mix": "onepass (2 B read : 4 + 1/16 B written per element)",
                           "GB/s": oc["GB/s"], "pattern": oc["pattern"],
                           "frac": round(achieved / oc["GB/s"], 4)}
    log("ceilings: " + ", ".join(f"{k} {v['GB/s']:.0f} ({v['pattern']})" for k, v in ceilings.items()))

    # ------------------------------------------------------------------
    # CPU oracle on a bounded sample (first cpu_rows rows, same arithmetic)
    # ------------------------------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        sample = np.ascontiguousarray(xb[:args.cpu_rows])
        se = sample.size
        log(f"cpu oracle on [{args.cpu_rows}, {cols}]")
        t = time.perf_counter()
        oq, os_ = orc.mxfp8_quantize_rowwise(sample)
        orc.mxfp8_quantize_colwise(sample)
        orc.mxfp8_dequantize(oq, os_, 1)
        dt = time.perf_counter() - t
        sbytes = 2 * se + se + se // 32 + se + ((args.cpu_rows + 31) // 32) * cols + 2 * se
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(sbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "host_cores": os.cpu_count(), "cpu_model": model,
               "sample": f"{args.cpu_rows} of {rows} rows of the same batch: row-wise + "
                         f"column-wise quantize and row-wise dequantize (the step's outputs), "
                         f"{dt:.1f} s single-threaded"}
        # the same oracle calls sharded by 32-row ranges over host threads (the
        # C calls release the GIL), for context next to the single-core figure
        import threading
        nthreads = max(1, min(16, os.cpu_count() or 1))
        chunk = ((args.cpu_rows + nthreads - 1) // nthreads + 31) // 32 * 32
        ranges = [(r, min(r + chunk, args.cpu_rows)) for r in range(0, args.cpu_rows, chunk)]

        def shard(r0, r1):
            xs = np.ascontiguousarray(sample[r0:r1])
            sq, ss = orc.mxfp8_quantize_rowwise(xs)
            orc.mxfp8_quantize_colwise(xs)
            orc.mxfp8_dequantize(sq, ss, 1)

        workers = [threading.Thread(target=shard, args=rg) for rg in ranges]
        t = time.perf_counter()
        for w in workers:
            w.start()
        for w in workers:
            w.join()
        dt_mt = time.perf_counter() - t
        cpu["all_threads"] = {"value": round(sbytes / dt_mt / 1e9, 4), "unit": "GB/s",
                              "cores": len(ranges), "seconds": round(dt_mt, 2)}

    # ------------------------------------------------------------------
    # breakdown: every other workload, timed on its own
    # ------------------------------------------------------------------
    breakdown = {}
    sq_ceilings = sq_ceilings_weight = None
    if not args.no_breakdown:
        def rotated(launches, nbytes, iters=20, mix=None):
            """Back-to-back launches cycling through copies with their own
            buffers; per-launch time = total / iters.  The untimed warm-up
            (warm_up) touches every copy and lasts at least WARM_S, so that no
            workload is timed while the GPU is still coming back from the
            host-side set-up before it.  With `mix`, the result also gives the
            fraction of that mix's streaming ceiling."""
            warm_up(lambda f: f(), launches)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(iters):
                launches[i % len(launches)]()
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_time(b) / iters
            gbs = nbytes / (ms * 1e-3) / 1e9
            r = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                 "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": int(nbytes),
                 "copies": len(launches)}
            if mix is not None:
                r["ceiling_mix"] = mix
                r["frac_ceiling"] = round(gbs / ceilings[mix]["GB/s"], 4)
            return r

        def ncopies(in_bytes):
            """Copies of a workload whose launch reads in_bytes, so that
            COLD_INPUT_BYTES of other copies pass between two reads of one."""
            return int(min(MAX_COPIES, max(2, -(-COLD_INPUT_BYTES // in_bytes) + 1)))

        # the main tensor, one output family at a time (same batches)
        rb = 2 * e + e + e // 32
        breakdown["act_16384 row-wise only"] = rotated(
            [lambda d=d: check(lib.mxq_quantize_rowwise(P(d["x"]), rows, cols, cols, P(d["qr"]),
                                                        cols, P(d["sr"]), cols // 32, None, 0, sp),
                               "rowwise") for d in batches], rb, mix="row")
        breakdown["act_16384 column-wise only"] = rotated(
            [lambda d=d: check(lib.mxq_quantize_colwise(P(d["x"]), rows, cols, P(d["qc"]),
                                                        P(d["sc"]), None, None, None, sp),
                               "colwise") for d in batches], 2 * e + e + batches[0]["sc"].numel(),
            mix="row")
        breakdown["act_16384 fake-quant only"] = rotated(
            [lambda d=d: check(lib.mxq_fake_quant(P(d["x"]), rows, cols, 1, P(d["fq"]), sp),
                               "fake_quant") for d in batches], 4 * e, mix="copy")

        def code_copies(qk, sk):
            """Copies of the batches' codes and scales for a dequantization
            (its input is half or less of a batch's), each with its own output."""
            in_bytes = batches[0][qk].numel() + batches[0][sk].numel()
            return [{"q": batches[i % BATCHES][qk].clone(), "s": batches[i % BATCHES][sk].clone(),
                     "out": torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)}
                    for i in range(ncopies(in_bytes))]

        # MXFP8 dequantization of the batches' codes, both axes
        for ax, qk, sk, nm in ((1, "qr", "sr", "row-wise"), (0, "qc", "sc", "column-wise")):
            dq = code_copies(qk, sk)
            breakdown[f"act_16384 {nm} dequantize"] = rotated(
                [lambda d=d, ax=ax: check(
                    lib.mxq_dequantize(P(d["q"]), P(d["s"]), rows, cols, ax, P(d["out"]), sp),
                    "dequantize") for d in dq], e + batches[0][sk].numel() + 2 * e, mix="dequant")
            del dq
        # column-wise in the transposed (backward-pass) layout, with and
        # without the row-wise outputs of the same pass
        breakdown["act_16384 one-pass, column-wise transposed"] = rotated(
            [lambda d=d: check(lib.mxq_quantize_colwise_t(P(d["x"]), rows, cols, P(d["qt"]), rows,
                                                          P(d["st"]), P(d["qr"]), P(d["sr"]),
                                                          P(d["fq"]), sp), "colwise_t")
             for d in batches], step_bytes, mix="onepass")
        # the same with qT rows QT_PAD bytes apart instead of `rows`: row
        # strides of a multiple of 4 KiB put the workgroups' concurrent
        # 128-byte column pieces on a subset of the memory channels
        breakdown[f"act_16384 one-pass, column-wise transposed, qT rows padded by {QT_PAD} B"] = rotated(
            [lambda d=d: check(lib.mxq_quantize_colwise_t(P(d["x"]), rows, cols, P(d["qt"]),
                                                          rows + QT_PAD, P(d["st"]), P(d["qr"]),
                                                          P(d["sr"]), P(d["fq"]), sp), "colwise_t")
             for d in batches], step_bytes, mix="onepass")
        breakdown["act_16384 column-wise transposed only"] = rotated(
            [lambda d=d: check(lib.mxq_quantize_colwise_t(P(d["x"]), rows, cols, P(d["qt"]), rows,
                                                          P(d["st"]), None, None, None, sp),
                               "colwise_t") for d in batches], 2 * e + e + e // 32, mix="row")
        # 1 x 128 block-FP8 (activation recipe) and its simulate-QAT
        b1 = 2 * e + e + 4 * (e // 128)
        breakdown["act_16384 block-FP8 1x128 quantize"] = rotated(
            [lambda d=d: check(lib.blockfp8_quantize_1x128(P(d["x"]), rows, cols, P(d["qr"]),
                                                           P(d["S1"]), None, sp), "bfp8 1x128")
             for d in batches], b1, mix="row")
        breakdown["act_16384 block-FP8 1x128 simulate-QAT (fake-quant only)"] = rotated(
            [lambda d=d: check(lib.blockfp8_fake_quant_1x128(P(d["x"]), rows, cols, P(d["fq"]),
                                                             sp), "bfp8 1x128 fq")
             for d in batches], 4 * e, mix="copy")
        # MXFP4 on the same batches: quantize, simulate-QAT, dequantize
        m4 = 2 * e + e // 2 + e // 32
        breakdown["act_16384 MXFP4 quantize"] = rotated(
            [lambda d=d: check(lib.mxfp4_quantize(P(d["x"]), rows, cols, P(d["q4"]), P(d["s4"]),
                                                  None, sp), "mxfp4") for d in batches], m4, mix="fp4")
        breakdown["act_16384 MXFP4 simulate-QAT (fake-quant only)"] = rotated(
            [lambda d=d: check(lib.mxfp4_fake_quant(P(d["x"]), rows, cols, P(d["fq"]), sp),
                               "mxfp4 fq") for d in batches], 4 * e, mix="copy")
        dq = code_copies("q4", "s4")
        breakdown["act_16384 MXFP4 dequantize"] = rotated(
            [lambda d=d: check(lib.mxfp4_dequantize(P(d["q"]), P(d["s"]), rows, cols, P(d["out"]),
                                                    sp), "mxfp4 dq") for d in dq],
            e // 2 + e // 32 + 2 * e, mix="fp4dq")
        del batches, dq
        torch.cuda.empty_cache()

        # weight [4097, 7168] row-wise (pad-then-crop case)
        wb = workloads.weight_4097()
        w0 = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev)
        wr, wc = wb.shape
        wbytes = 3 * wr * wc + wr * wc // 32
        wsets = [(w0.clone(), torch.empty((wr, wc), dtype=torch.uint8, device=dev),
                  torch.empty((wr, wc // 32), dtype=torch.uint8, device=dev))
                 for _ in range(ncopies(wr * wc * 2))]
        breakdown["weight_4097 row-wise"] = rotated(
            [lambda t=t: check(lib.mxq_quantize_rowwise(P(t[0]), wr, wc, wc, P(t[1]), wc, P(t[2]),
                                                        wc // 32, None, 0, sp), "rowwise")
             for t in wsets], wbytes, mix="row")
        # the row-wise mix's streams on these buffers (the codes buffer stands
        # in for the planes that mix does not write)
        wc_ceil, _ = measure_ceilings(load_streams(), [{"x": t[0], "qc": t[1], "qr": t[1], "fq": t[1],
                                                        "sr": t[2]} for t in wsets],
                                      wr, wc, stream, sp, mixes=("row",))
        breakdown["weight_4097 row-wise"]["ceiling_same_size_mix"] = "row"
        breakdown["weight_4097 row-wise"]["frac_ceiling_same_size"] = round(
            breakdown["weight_4097 row-wise"]["GB/s"] / wc_ceil["row"]["GB/s"], 4)
        sq_ceilings_weight = wc_ceil
        del w0, wsets

        # mx_small row-wise + dequantize: a latency measurement (the data is
        # cache-resident at this size whatever is done)
        mb = workloads.mx_small()
        m = torch.from_numpy(mb.view(np.int16)).view(torch.bfloat16).to(dev)
        mq = torch.empty(mb.shape, dtype=torch.uint8, device=dev)
        ms_ = torch.empty((mb.shape[0], mb.shape[1] // 32), dtype=torch.uint8, device=dev)
        md = torch.empty(mb.shape, dtype=torch.bfloat16, device=dev)
        me = mb.size
        breakdown["mx_small row-wise"] = rotated(
            [lambda: check(lib.mxq_quantize_rowwise(P(m), mb.shape[0], mb.shape[1], mb.shape[1],
                                                    P(mq), mb.shape[1], P(ms_), mb.shape[1] // 32,
                                                    None, 0, sp), "rowwise")], 3 * me + me // 32)
        breakdown["mx_small dequantize"] = rotated(
            [lambda: check(lib.mxq_dequantize(P(mq), P(ms_), mb.shape[0], mb.shape[1], 1, P(md),
                                              sp), "dequantize")], 3 * me + me // 32)

        # grouped MoE experts: 384 tensors (11.3 GB in), one launch
        shapes = workloads.moe_shapes()
        mult = workloads.moe_multipliers()
        log("generating moe_experts (384 tensors)")
        xs = [workloads.moe_tensor(i, r, c, mult[i // 3], dev) for i, (_, r, c) in enumerate(shapes)]
        outs = [(torch.empty((r, c), dtype=torch.uint8, device=dev),
                 torch.empty((r, c // 32), dtype=torch.uint8, device=dev)) for (_, r, c) in shapes]
        descs = (mxq.GroupDesc * len(xs))()
        for i, (t, (q_, s_)) in enumerate(zip(xs, outs)):
            descs[i] = mxq.GroupDesc(t.data_ptr(), q_.data_ptr(), s_.data_ptr(), t.shape[0],
                                     t.shape[1], t.shape[1], t.shape[1], t.shape[1] // 32)
        wsz = lib.mxq_grouped_workspace_size(len(xs))
        gws = torch.empty(wsz, dtype=torch.uint8, device=dev)
        ge = sum(r * c for (_, r, c) in shapes)
        breakdown["moe_experts grouped row-wise"] = rotated(
            [lambda: check(lib.mxq_quantize_rowwise_grouped(descs, len(xs), P(gws), wsz, sp),
                           "grouped")], 3 * ge + ge // 32, iters=10, mix="row")
        del outs, gws
        torch.cuda.empty_cache()
        # NVFP4 of the 256 gate/up tensors in one grouped call, gate and up of
        # an expert sharing one global scale (the exported weight_scale_2)
        gu = [i for i, (name, _, _) in enumerate(shapes)
              if name.endswith(("gate_proj.weight", "up_proj.weight"))]
        assert len(gu) == 2 * (len(shapes) // 3)
        nvd = (mxq.NvGroupDesc * len(gu))()
        nv_outs = []
        for k, i in enumerate(gu):
            t = xs[i]
            q_ = torch.empty((t.shape[0], t.shape[1] // 2), dtype=torch.uint8, device=dev)
            s_ = torch.empty((t.shape[0], t.shape[1] // 16), dtype=torch.uint8, device=dev)
            nv_outs.append((q_, s_))
            nvd[k] = mxq.NvGroupDesc(t.data_ptr(), q_.data_ptr(), s_.data_ptr(), t.shape[0],
                                     t.shape[1], i // 3, 0)
        n_exp = len(shapes) // 3
        nvg = torch.empty((n_exp,), dtype=torch.float32, device=dev)
        nvw_n = lib.nvfp4_grouped_workspace_size(nvd, len(gu))
        nvw = torch.empty((nvw_n,), dtype=torch.uint8, device=dev)
        gue = sum(xs[i].numel() for i in gu)
        breakdown["moe gate/up NVFP4 grouped, shared scale per expert (unique bytes)"] = rotated(
            [lambda: check(lib.nvfp4_quantize_grouped(nvd, len(gu), P(nvg), n_exp, P(nvw), nvw_n,
                                                      sp), "nvfp4 grouped")],
            2 * gue + gue // 2 + gue // 16 + 4 * n_exp, iters=10)
        # its amax pass reads every tensor (the read-only mix), its encoding
        # pass reads them again and writes codes and scales (the FP4-encode
        # mix): the two act_16384 streams back to back bound the pair
        r = breakdown["moe gate/up NVFP4 grouped, shared scale per expert (unique bytes)"]
        two = (2 * gue / ceilings["read"]["GB/s"] + (2 * gue + gue // 2 + gue // 16)
               / ceilings["fp4"]["GB/s"]) / 1e3
        r["two_stream_us"] = round(two, 2)
        r["frac_two_stream"] = round(two / r["us"], 4)
        r["two_stream_on"] = "act_16384 batches"
        del xs, nv_outs, nvw
        torch.cuda.empty_cache()

        # square [8192, 8192]: block-FP8 and NVFP4, quantize and dequantize
        yb = workloads.square_8192()
        y0 = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).to(dev)
        n_ = yb.shape[0]
        ye = yb.size
        nwsz = lib.nvfp4_workspace_size()
        bbytes = 3 * ye + 4 * (n_ // 128) ** 2
        nbytes = 2 * ye + ye // 2 + ye // 16 + 4
        # as many copies as the smallest input (NVFP4 dequantization's) needs;
        # each workload cycles over as many as its own input needs (more copies
        # than that measured slower, though no copy is re-read sooner)
        ysets = []
        for _ in range(ncopies(ye // 2 + ye // 16)):
            ysets.append({
                "y": y0.clone(),
                "bq": torch.empty((n_, n_), dtype=torch.uint8, device=dev),
                "bS": torch.empty((n_ // 128, n_ // 128), dtype=torch.float32, device=dev),
                "bd": torch.empty((n_, n_), dtype=torch.bfloat16, device=dev),
                "rq8": torch.empty((n_, n_), dtype=torch.uint8, device=dev),
                "rs8": torch.empty((n_, n_ // 32), dtype=torch.uint8, device=dev),
                "nq": torch.empty((n_, n_ // 2), dtype=torch.uint8, device=dev),
                "ns": torch.empty((n_, n_ // 16), dtype=torch.uint8, device=dev),
                "ng": torch.empty((1,), dtype=torch.float32, device=dev),
                "nws": torch.empty((nwsz,), dtype=torch.uint8, device=dev)})
        del y0
        # the dequantizers and the FP8 -> MXFP8 pass read codes and scales of
        # every copy: quantize every copy once, untimed
        for d in ysets:
            check(lib.blockfp8_quantize(P(d["y"]), n_, n_, 128, P(d["bq"]), P(d["bS"]), sp), "bfp8")
            check(lib.nvfp4_quantize(P(d["y"]), n_, n_, P(d["nq"]), P(d["ns"]), P(d["ng"]),
                                     P(d["nws"]), nwsz, sp), "nvfp4")
        torch.cuda.synchronize()
        breakdown["square_8192 block-FP8 quantize"] = rotated(
            [lambda d=d: check(lib.blockfp8_quantize(P(d["y"]), n_, n_, 128, P(d["bq"]), P(d["bS"]),
                                                     sp), "bfp8") for d in ysets[:ncopies(2 * ye)]],
            bbytes, mix="row")
        breakdown["square_8192 block-FP8 dequantize"] = rotated(
            [lambda d=d: check(lib.blockfp8_dequantize(P(d["bq"]), P(d["bS"]), n_, n_, 128,
                                                       P(d["bd"]), sp), "bfp8 dq")
             for d in ysets[:ncopies(ye + 4 * (n_ // 128) ** 2)]], bbytes, mix="dequant")
        breakdown["square_8192 block-FP8 -> MXFP8 re-quantize (one pass)"] = rotated(
            [lambda d=d: check(lib.blockfp8_to_mxfp8(P(d["bq"]), P(d["bS"]), n_, n_, 128,
                                                     P(d["rq8"]), P(d["rs8"]), sp), "requant")
             for d in ysets[:ncopies(ye + 4 * (n_ // 128) ** 2)]],
            ye + 4 * (n_ // 128) ** 2 + ye + ye // 32, mix="requant")
        breakdown["square_8192 NVFP4 quantize (unique bytes)"] = rotated(
            [lambda d=d: check(lib.nvfp4_quantize(P(d["y"]), n_, n_, P(d["nq"]), P(d["ns"]),
                                                  P(d["ng"]), P(d["nws"]), nwsz, sp), "nvfp4")
             for d in ysets[:ncopies(2 * ye)]], nbytes)
        breakdown["square_8192 NVFP4 dequantize"] = rotated(
            [lambda d=d: check(lib.nvfp4_dequantize(P(d["nq"]), P(d["ns"]), P(d["ng"]), n_, n_,
                                                    P(d["bd"]), sp), "nvfp4 dq") for d in ysets],
            nbytes, mix="fp4dq")
        # the same streams on the square_8192 buffers, run last since they
        # overwrite codes: the square kernels also stand against ceilings
        # measured at their own size (about half the bytes per launch of the
        # act_16384 streams, so ramp-up and drain weigh the same for both)
        sq_batches = [{"x": d["y"], "qc": d["bq"], "qr": d["rq8"], "fq": d["bd"], "sr": d["rs8"]}
                      for d in ysets[:ncopies(2 * ye)]]
        sq_ceilings, _ = measure_ceilings(load_streams(), sq_batches, n_, n_, stream, sp)
        for key, mix in (("square_8192 block-FP8 quantize", "row"),
                         ("square_8192 block-FP8 dequantize", "dequant"),
                         ("square_8192 block-FP8 -> MXFP8 re-quantize (one pass)", "requant"),
                         ("square_8192 NVFP4 dequantize", "fp4dq")):
            r = breakdown[key]
            r["ceiling_same_size_mix"] = mix
            r["frac_ceiling_same_size"] = round(r["GB/s"] / sq_ceilings[mix]["GB/s"], 4)
        # NVFP4 quantize: its amax pass reads x (the read-only mix), its
        # encoding pass reads x again and writes codes and scales (the FP4
        # encode mix); the two streams back to back bound the pair of passes
        r = breakdown["square_8192 NVFP4 quantize (unique bytes)"]
        two = (2 * ye / sq_ceilings["read"]["GB/s"] + (2 * ye + ye // 2 + ye // 16)
               / sq_ceilings["fp4"]["GB/s"]) / 1e3
        r["two_stream_us"] = round(two, 2)
        r["frac_two_stream"] = round(two / r["us"], 4)
        r["two_stream_on"] = "square_8192 buffers"
        del ysets, sq_batches

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "act_16384: bf16 [16384, 7168], 0.5*Student-t(3), seed 3; MXFP8 "
                               "column-wise + row-wise + fused row-wise fake-quant in one pass",
                   "rows": rows, "cols": cols, "bytes_per_step": step_bytes,
                   "resident_batches": BATCHES,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceilings": ceilings,
        "ceilings_square_8192": sq_ceilings,
        "ceilings_weight_4097": sq_ceilings_weight,
        "ceiling_runs": ceiling_runs,
        "breakdown": breakdown,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
