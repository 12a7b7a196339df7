#!/usr/bin/env python3
"""Benchmark: nested NF4 -> FP16 dequantization of a 28672 x 8192 weight, bs 64.

One step is one call of dq4_nested_dequant over the whole tensor (235 M
elements): element -> block -> group indexing, metadata fetch, in-register
scale reconstruction, 4-bit decode and FP16 conversion and store, all in one
kernel.  Inputs are resident in HBM before the timed region starts.  Several
independent input/output buffer sets are cycled so repeated steps cannot be
served from the 256 MB last-level cache.

Prints ONE JSON line (rank 0, one GPU):
  value      = algorithmic bytes per step / wall-clock time per step, in GB/s
  roofline   = the kernel's achieved bandwidth from HIP events on its stream
               against MI355X's 8 TB/s HBM peak, and the HBM traffic measured
               by rocprofv3 counters (profiles/), while the built kernel's
               instruction digest matches the one the counters were taken on
  attainable = the library's memory twin of the kernel (same tiles, loads and
               stores, no arithmetic) timed on the same buffers: the ceiling
               of this access pattern on the GPU at hand
  cpu_baseline = the CPU oracle on the same inputs, on the host's threads over
               disjoint element ranges (single_core inside: on one thread)
Timing protocol after the bitsandbytes issue's evidence plan ("B300 evidence
plan"): >= 20 warmups; the timed region is K launches between one pair of
events; right after it the same K launches run again in 7 batches with an
event pair each, and every batch sample is reported with median, p10 and p90
(kernel_us.batches_after).  The batch events stay out of the timed region
because an event recorded between two launches holds the second one back
until its timestamp is written.  Whatever --warmup asks for, at least 20
untimed launches and 0.1 s of them run before each timed region
(warmup_launches in the JSON line counts them): the first milliseconds of a
burst of launches run slower while the GPU's clocks settle.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dequantized GB/s (fraction of HBM peak), NF4→FP16 28672×8192 bs64"
HBM_PEAK_GBS = 8000.0
MATRIX_PEAK_16BIT = 2500.0   # TFLOP/s, dense FP16/BF16 matrix cores (no sparsity)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "dq4_tile_kernel_f16_28672x8192_bs64_pmc.json")
KERNEL_DIGESTS = os.path.join(ROOT, "block_wise_bit_amd", "libdq4_kernels.json")
HEADLINE_KERNEL = "_ZN3dq412_GLOBAL__N_115dq4_tile_kernelILi1EEEvNS0_4ArgsEll"


def host_threads() -> int:
    """Threads for the CPU oracle: the machine's CPU share, whatever os.cpu_count() reports."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_dequant_threaded(x, first: int, count: int, dt_name: str, threads: int):
    """The C oracle over elements [first, first + count) of the inputs x,
    split into `threads` disjoint element ranges run concurrently (the oracle
    releases the GIL while it runs).  Returns (output as the oracle gives it:
    uint16 bits for FP16/BF16, float32 for FP32; seconds of wall clock)."""
    import concurrent.futures

    import numpy as np

    import oracle

    out = np.empty(count, dtype=np.float32 if dt_name == "f32" else np.uint16)
    chunk = -(-count // threads) if count else 1
    chunk += (-chunk) % 8

    def one(start):
        c = min(chunk, count - start)
        out[start:start + c] = oracle.dequant_range(
            x.packed, x.scale_codes, x.nested_absmax, x.scale_codebook, x.codebook4,
            x.offset, first + start, c, x.blocksize, x.nested_blocksize, dt_name)

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(one, range(0, count, chunk)))
    return out, time.perf_counter() - t0


def device_bits(t):
    """A device tensor's values as host bits (uint16 for 16-bit types, float32 otherwise)."""
    import numpy as np
    import torch
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def algorithmic_bytes(n: int, blocksize: int, out_bytes: int, nested: int = 256) -> int:
    """Bytes the method must move once: packed nibbles, codes, absmax, codebooks, output."""
    nb = -(-n // blocksize)
    ng = -(-nb // nested)
    return (n + 1) // 2 + nb + 4 * ng + 4 * (256 + 16) + out_bytes * n


def kernel_digest(symbol: str = HEADLINE_KERNEL):
    """Instruction digest of the built kernel (written by the library build)."""
    try:
        with open(KERNEL_DIGESTS) as fh:
            return json.load(fh).get(symbol)
    except (OSError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if the
    counters were taken on exactly the kernel code built now; else None."""
    try:
        with open(PMC_SUMMARY) as fh:
            s = json.load(fh)
    except (OSError, ValueError):
        return None
    digest = kernel_digest(s.get("kernel_symbol", HEADLINE_KERNEL))
    if digest is None or s.get("kernel_isa_sha256_16") != digest:
        return None
    return s.get("hbm_bytes_per_launch")


def run_env(torch) -> dict:
    """Identity of what ran: software versions, the GPU, and a digest of the
    library binary (the kernel digests identify each kernel's code)."""
    import hashlib
    lib = os.path.join(ROOT, "block_wise_bit_amd", "libdq4.so")
    try:
        with open(lib, "rb") as fh:
            lib_digest = hashlib.sha256(fh.read()).hexdigest()[:16]
    except OSError:
        lib_digest = None
    props = torch.cuda.get_device_properties(0)
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "library_sha256_16": lib_digest, "python": platform.python_version(),
            "host_logical_cpus": os.cpu_count()}


# Untimed launches before any timed region, whatever --warmup asks for: at
# least this many launches and this much GPU time.  MI355X runs the first
# milliseconds of a burst of launches slower while its clocks settle, and the
# bitsandbytes issue's evidence plan ("B300 evidence plan") asks for >= 20
# warmup launches.
WARMUP_MIN_LAUNCHES = 20
WARMUP_MIN_SECONDS = 0.1


def warm_up(step, asked: int, torch) -> int:
    """Run step(k) for k = 0, 1, ... until at least max(asked, 20) launches
    and 0.1 s have gone by (synchronizing every 20 launches); returns the
    number of launches."""
    want = max(int(asked), WARMUP_MIN_LAUNCHES)
    k = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(WARMUP_MIN_LAUNCHES):
            step(k)
            k += 1
        torch.cuda.synchronize()
        if k >= want and time.perf_counter() - t0 >= WARMUP_MIN_SECONDS:
            return k


def timed_region(step, K: int, stream, torch):
    """K calls of step(k) between one pair of events on `stream`, with
    torch.cuda.synchronize() and the wall clock on both sides; returns (device
    microseconds per step from the events, wall seconds for the region)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(K):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) * 1e3 / K, wall


def timed_batches(step, per, stream, torch, first: int = 0):
    """Consecutive batches of per[i] calls of step(k), k counting on from
    `first`, each between its own pair of events; returns microseconds per
    call for every batch."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in per]
    torch.cuda.synchronize()
    k = first
    for (e0, e1), m in zip(evs, per):
        e0.record(stream)
        for _ in range(m):
            step(k)
            k += 1
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 / m for (e0, e1), m in zip(evs, per)]


def raw_dequant_steps(dq4, sets, offset, n, bs, out_code, stream):
    """step(k): dq4_nested_dequant on buffer set k mod len(sets), called
    through the C ABI with the arguments the checked wrapper already accepted
    for that set.  Raises on a non-OK status."""
    import ctypes
    lib = dq4.library()
    handle = ctypes.c_void_p(stream.cuda_stream)
    calls = [(dev["packed"].data_ptr(), dev["scale_codes"].data_ptr(),
              dev["nested_absmax"].data_ptr(), dev["scale_codebook"].data_ptr(),
              dev["codebook4"].data_ptr(), ctypes.c_float(offset), n, bs, 256, out_code,
              out.data_ptr(), handle) for dev, out in sets]

    def step(k):
        st = lib.dq4_nested_dequant(*calls[k % len(calls)])
        if st != dq4.DQ4_OK:
            raise RuntimeError(f"dq4_nested_dequant: {dq4.dq4_status_string(st)}")
    return step


def raw_twin_steps(dq4, sets, n, stream):
    """The same for the memory twin."""
    import ctypes
    lib = dq4.library()
    handle = ctypes.c_void_p(stream.cuda_stream)
    calls = [(dev["packed"].data_ptr(), n, out.data_ptr(), handle) for dev, out in sets]

    def step(k):
        st = lib.dq4_memory_twin_f16(*calls[k % len(calls)])
        if st != dq4.DQ4_OK:
            raise RuntimeError(f"dq4_memory_twin_f16: {dq4.dq4_status_string(st)}")
    return step


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def copy_calibration(args, torch) -> int:
    """A plain copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel over
    its true bytes give the scale factors of the HBM byte counters."""
    nbytes = args.copy_calibration << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "us_per_copy": round(us, 3),
                      "GBps": round(2 * nbytes / (us * 1e-6) / 1e9, 2)}), flush=True)
    return 0


# MI355X's last-level (Infinity) cache holds 256 MB.  Cycling less packed
# input than that lets calls read their weight from the cache (measured: small
# shapes up to ~15 % faster), which times the cache, not HBM.
COLD_PACKED_BYTES = 600_000_000
PRIMARY_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008), (8192, 8192), (28672, 8192))


def compare_unfused(args, torch, dq4, inputs) -> int:
    """Fused single kernel vs the unfused three-launch sequence on the primary
    standalone matrix of the bitsandbytes issue's evidence plan: NF4 and FP4,
    FP16 and BF16 (FP32 as control), block size 64, five weight shapes.
    Baseline and candidate are interleaved batch by batch; each cell cycles
    enough buffer sets that no set is reused within ~1 GB of traffic and
    that the packed inputs cycled exceed COLD_PACKED_BYTES, so every call
    reads its packed weight from HBM, not from the last-level cache."""
    import math

    import numpy as np

    all_dtypes = (("f16", torch.float16, 2), ("bf16", torch.bfloat16, 2),
                  ("f32", torch.float32, 4))
    # the primary matrix, then the odd-tail control (1-D, odd length: a packed
    # tail nibble, a partial outer block and a partial nested group)
    cases = [(rows, cols, all_dtypes, None) for rows, cols in PRIMARY_SHAPES]
    cases.append((1, inputs.TAIL_SWEEP_N, all_dtypes[:1], "odd_tail"))
    cells = []
    for rows, cols, dtypes, control in cases:
        n = rows * cols
        for fmt in ("nf4", "fp4"):
            x = inputs.make_inputs(n, 64, fmt, -0.02, seed=inputs.SEED_BASE + 2, n_rows=rows,
                                   n_cols=cols)
            for dt, tdt, ob in dtypes:
                alg = algorithmic_bytes(n, 64, ob)
                n_sets = max(2, math.ceil(1.2e9 / alg),
                             math.ceil(COLD_PACKED_BYTES / ((n + 1) // 2)))
                ws_len = dq4.dq4_unfused_workspace_bytes(n, 64) // 4
                sets = [(dq4.to_device(x, "cuda:0"), torch.empty(n, dtype=tdt, device="cuda:0"),
                         torch.empty(ws_len, dtype=torch.float32, device="cuda:0"))
                        for _ in range(n_sets)]
                stream = torch.cuda.current_stream()

                # both launch on torch's current stream (the capture stream while a
                # graph is being captured)
                def fused(k):
                    dev, out, _ = sets[k % n_sets]
                    dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=64,
                                           out_dtype=tdt, out=out)

                def unfused(k):
                    dev, out, ws = sets[k % n_sets]
                    dq4.dq4_nested_dequant_unfused(**dev, offset=float(x.offset), n=n,
                                                   blocksize=64, out_dtype=tdt, out=out,
                                                   scale_workspace=ws)

                for k in range(args.warmup):
                    fused(k)
                    unfused(k)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for k in range(5):
                    fused(k)
                e1.record(stream)
                torch.cuda.synchronize()
                inner = max(5, int(2000.0 / max(e0.elapsed_time(e1) * 1e3 / 5, 1.0)))

                # device time: `inner` calls captured in one HIP graph and replayed,
                # so host-side launch cost is out and only the GPU's work and its
                # inter-kernel gaps remain
                graphs = {}
                for name, fn in (("fused", fused), ("unfused", unfused)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for k in range(inner):
                            fn(k)
                    g.replay()
                    graphs[name] = g
                torch.cuda.synchronize()

                def timed(run):
                    a, b = (torch.cuda.Event(enable_timing=True),
                            torch.cuda.Event(enable_timing=True))
                    a.record(torch.cuda.current_stream())
                    run()
                    b.record(torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    return a.elapsed_time(b) * 1e3 / inner

                samples = {"fused": [], "unfused": [], "fused_eager": [], "unfused_eager": []}
                for _ in range(max(7, args.batches)):   # baseline and candidate interleaved
                    for name in ("fused", "unfused"):
                        samples[name].append(timed(graphs[name].replay))
                    for name, fn in (("fused_eager", fused), ("unfused_eager", unfused)):
                        samples[name].append(timed(lambda: [fn(k) for k in range(inner)]))
                del graphs
                # the two paths must agree bit for bit on this cell
                dev0, out0, ws0 = sets[0]
                ref = dq4.dq4_nested_dequant(**dev0, offset=float(x.offset), n=n, blocksize=64,
                                             out_dtype=tdt)
                dq4.dq4_nested_dequant_unfused(**dev0, offset=float(x.offset), n=n, blocksize=64,
                                               out_dtype=tdt, out=out0, scale_workspace=ws0)
                iview = torch.int32 if ob == 4 else torch.int16
                bit_equal = bool(torch.equal(ref.view(iview), out0.view(iview)))
                oracle_cell = None
                if not args.no_cpu:
                    # the oracle beside it: timed over the whole tensor, and the
                    # fused output compared with it bit for bit
                    want, t_cpu = oracle_dequant_threaded(x, 0, n, dt, host_threads())
                    hv = np.uint32 if ob == 4 else np.uint16
                    oracle_cell = {
                        "seconds": round(t_cpu, 4), "cores": host_threads(),
                        "GBps": round(alg / t_cpu / 1e9, 3),
                        "mismatches": int(np.count_nonzero(device_bits(ref).view(hv)
                                                           != want.view(hv)))}
                    del want
                del ref
                med = {k: percentile(v, 0.5) for k, v in samples.items()}
                f_med, u_med = med["fused"], med["unfused"]
                cell = {"shape": f"{rows}x{cols}" if control is None else f"n={n}",
                        "control": control, "format": fmt, "out": dt,
                        "fused_us": round(f_med, 2), "unfused_us": round(u_med, 2),
                        "speedup": round(u_med / f_med, 4),
                        "fused_p10_p90": [round(percentile(samples["fused"], q), 2)
                                          for q in (0.1, 0.9)],
                        "unfused_p10_p90": [round(percentile(samples["unfused"], q), 2)
                                            for q in (0.1, 0.9)],
                        "fused_GBps": round(alg / (f_med * 1e-6) / 1e9, 1),
                        "fused_frac": round(alg / (f_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        # the unfused form also writes, rewrites and rereads the FP32
                        # scale buffer: 16 more bytes per block
                        "unfused_algorithmic_bytes": alg + 16 * (-(-n // 64)),
                        "unfused_frac": round((alg + 16 * (-(-n // 64))) / (u_med * 1e-6) / 1e9
                                              / HBM_PEAK_GBS, 4),
                        "eager_fused_us": round(med["fused_eager"], 2),
                        "eager_unfused_us": round(med["unfused_eager"], 2),
                        "eager_speedup": round(med["unfused_eager"] / med["fused_eager"], 4),
                        "samples_us": {k: [round(x, 2) for x in v] for k, v in samples.items()},
                        "buffer_sets": n_sets, "inner": inner, "bit_equal": bit_equal,
                        "oracle": oracle_cell}
                cells.append(cell)
                print(f"[compare] {cell['shape']} {fmt} {dt}: fused {f_med:.2f} us, "
                      f"unfused {u_med:.2f} us, x{u_med / f_med:.3f} (eager "
                      f"{cell['eager_fused_us']:.2f} / {cell['eager_unfused_us']:.2f} us)",
                      file=sys.stderr, flush=True)
                del sets
                torch.cuda.empty_cache()

    def geomean(vals):
        return math.exp(sum(math.log(v) for v in vals) / len(vals))

    main = [c for c in cells if c["control"] is None]
    primary = [c["speedup"] for c in main if c["out"] in ("f16", "bf16")]
    controls = [c["speedup"] for c in main if c["out"] == "f32"]
    eager = [c["eager_speedup"] for c in main if c["out"] in ("f16", "bf16")]
    odd_tail = {c["format"]: c["speedup"] for c in cells if c["control"] == "odd_tail"}
    all_equal = all(c["bit_equal"] for c in cells)
    if not args.no_cpu:
        all_equal = all_equal and all(c["oracle"]["mismatches"] == 0 for c in cells)
    print(json.dumps({
        "metric": "fused vs unfused nested dequant speedup, geomean over NF4/FP4 x FP16/BF16, "
                  "bs64, primary standalone matrix",
        "value": round(geomean(primary), 4), "unit": "x", "higher_is_better": True,
        "fp32_control_geomean": round(geomean(controls), 4),
        "odd_tail_control_speedup": odd_tail,
        "eager_geomean": round(geomean(eager), 4),
        "timing": "device time per call from HIP-graph replays of `inner` calls, median of "
                  ">= 7 interleaved batches; eager_* = the same calls launched from Python",
        "min_primary_speedup": round(min(primary), 4),
        "fused_equals_unfused_bitwise": all(c["bit_equal"] for c in cells),
        "fused_equals_oracle_bitwise": None if args.no_cpu else
            all(c["oracle"]["mismatches"] == 0 for c in cells),
        "n_gpus": 1, "warmup": args.warmup, "data": "synthetic", "cells": cells,
        "device": torch.cuda.get_device_name(0), "env": run_env(torch)}), flush=True)
    return 0 if all_equal else 3


def out_prod_bench(args, torch, dq4, inputs) -> int:
    """out_prod of the 151936 x 5376 NF4 output head against a src1 of m
    rows per weight row (the LoRA backward of the output head in the
    llama.cpp PR), by both routes:
    * row-blocked: 13 F32 windows of <= 256 MiB, one FP32 library GEMM each
      (also timed: the windows' dequantization alone, and the single-window
      whole copy);
    * fused: the weight decoded inside an FP32 matrix-core GEMM, no window.
    The two results must agree within twice the FP32 summation bound."""
    wl = inputs.OUTPUT_HEAD
    x = wl.inputs()
    dev = dq4.to_device(x, "cuda:0")
    m = args.out_prod_m
    g = torch.Generator(device="cuda:0").manual_seed(7)
    src1 = torch.randn((wl.n_rows, m), dtype=torch.float32, device="cuda:0", generator=g)
    # with --out-prod-transposed the routes get the same values stored m x n_rows
    transposed = bool(args.out_prod_transposed)
    src1_arg = src1.t().contiguous() if transposed else src1
    dst = torch.empty((m, wl.n_cols), dtype=torch.float32, device="cuda:0")
    budget = 256 << 20
    rows_pb = dq4.dq4_rows_per_block(wl.n_cols, 4, budget)
    ws = torch.empty(rows_pb * wl.n_cols, dtype=torch.float32, device="cuda:0")
    windows = dq4.dq4_row_windows(wl.n_rows, wl.n_cols, 4, budget)
    flops = 2.0 * m * wl.n_rows * wl.n_cols
    fused_ws_bytes = dq4.dq4_out_prod_fused_workspace_bytes(wl.n_rows, wl.n_cols, m,
                                                            src1_transposed=transposed)
    fused_ws = torch.empty(max(fused_ws_bytes // 4, 0), dtype=torch.float32, device="cuda:0")
    kw = dict(offset=float(x.offset), n_rows=wl.n_rows, n_cols=wl.n_cols, blocksize=64,
              src1=src1_arg, src1_transposed=transposed)

    def timeit(fn, reps):
        # each route is warmed on its own before it is timed: at least 20
        # calls and 0.1 s of them (the GPU's clocks after the previous
        # route's different load take a while to settle; measured: the fused
        # route at m = 64 took 1.10 ms over 7 calls right after the blocked
        # route, 0.94 ms once warmed)
        warm_up(lambda k: fn(), 0, torch)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps  # ms

    def blocked():
        dq4.dq4_out_prod_rows(**dev, **kw, dst=dst, workspace=ws)

    def fused():
        dq4.dq4_out_prod_fused(**dev, **kw, dst=dst, workspace=fused_ws)

    def windows_only():
        for r0, rows in windows:
            dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=wl.n_rows,
                                        n_cols=wl.n_cols, r0=r0, rows=rows, blocksize=64,
                                        out_dtype=torch.float32, out=ws)

    reps = max(20, args.steps // 35)
    t_blocked = timeit(blocked, reps)
    out_blocked = dst.clone()
    t_fused = timeit(fused, reps)
    out_fused = dst.clone()
    t_dequant = timeit(windows_only, reps)
    whole = torch.empty(wl.n_rows * wl.n_cols, dtype=torch.float32, device="cuda:0")

    def whole_copy():
        dq4.dq4_out_prod_rows(**dev, **kw, dst=dst, workspace=whole)

    t_whole = timeit(whole_copy, reps)
    del whole
    scale = out_blocked.abs().max().clamp_min(1e-30)
    rel_whole = float((dst - out_blocked).abs().max() / scale)
    rel_fused = float((out_fused - out_blocked).abs().max() / scale)
    tflops = {name: round(flops / (t * 1e-3) / 1e12, 2)
              for name, t in (("fused", t_fused), ("blocked", t_blocked), ("whole", t_whole))}
    best = max(tflops.values())
    cpu, sampled = None, None
    if not args.no_cpu:
        # the oracle beside it, on a bounded sample: the first row window is a
        # weight of its own (rows 0 .. rows_pb - 1, the prefix of every array).
        # The fused route runs on it; the oracle dequantizes it and numpy sums
        # the products in float64; the fused result must lie within the FP32
        # summation bound gamma_K * sum |src1| |w| of that float64 sum.
        import numpy as np
        rows_s = rows_pb
        dst_s = torch.empty((m, wl.n_cols), dtype=torch.float32, device="cuda:0")
        dq4.dq4_out_prod_fused(**dev, offset=float(x.offset), n_rows=rows_s, n_cols=wl.n_cols,
                               blocksize=64,
                               src1=src1_arg[:, :rows_s] if transposed else src1[:rows_s],
                               src1_transposed=transposed, dst=dst_s)
        got_s = dst_s.cpu().numpy().astype(np.float64)
        a_s = src1[:rows_s].cpu().numpy().astype(np.float64)
        w_s, t_deq = oracle_dequant_threaded(x, 0, rows_s * wl.n_cols, "f32", host_threads())
        w_s = w_s.reshape(rows_s, wl.n_cols).astype(np.float64)
        t0 = time.perf_counter()
        ref = a_s.T @ w_s
        t_mm = time.perf_counter() - t0
        bound = np.abs(a_s).T @ np.abs(w_s)
        k = float(rows_s) * 2.0 ** -24
        excess = np.abs(got_s - ref) / np.maximum(k / (1 - k) * bound, 1e-300)
        sample_flops = 2.0 * m * rows_s * wl.n_cols
        cpu = {"value": round(sample_flops / (t_deq + t_mm) / 1e12, 5), "unit": "TFLOP/s",
               "cores": host_threads(), "kind": "oracle",
               "sample": f"rows 0..{rows_s - 1} of {wl.n_rows} (the first row window), m = {m}: "
                         f"the C oracle's dequantization on {host_threads()} threads "
                         f"({t_deq:.2f} s) then numpy's float64 product ({t_mm:.2f} s)"}
        sampled = {"rows": rows_s, "max_error_over_fp32_bound": float(f"{float(excess.max()):.3g}"),
                   "within_bound": bool(excess.max() <= 1.0)}
        del a_s, w_s, ref, bound, got_s, dst_s
    print(json.dumps({
        "metric": "out_prod of the 151936x5376 NF4 output head, FP32 TFLOP/s (fused route)",
        "value": tflops["fused"], "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1,
        "data": "synthetic",
        "config": {"workload": wl.name, "m": m, "src1_transposed": transposed,
                   "windows": len(windows),
                   "rows_per_window": rows_pb, "transient_bytes": rows_pb * wl.n_cols * 4,
                   "fused_workspace_bytes": fused_ws_bytes},
        "ms_fused": round(t_fused, 4), "ms_blocked": round(t_blocked, 4),
        "ms_dequant_windows": round(t_dequant, 4),
        "dequant_share_of_blocked": round(t_dequant / t_blocked, 4),
        "ms_whole_copy": round(t_whole, 4), "whole_copy_transient_bytes":
            wl.n_rows * wl.n_cols * 4,
        "TFLOPs": tflops, "fused_speedup_vs_blocked": round(t_blocked / t_fused, 3),
        "blocked_vs_whole_max_rel_diff": rel_whole, "fused_vs_blocked_max_rel_diff": rel_fused,
        "roofline": {"bound": "mfma", "achieved": tflops["fused"], "peak": 157.3,
                     "unit": "TFLOP/s", "frac": round(tflops["fused"] / 157.3, 4)},
        "best_route_TFLOPs": best, "cpu_baseline": cpu, "sampled_parity": sampled,
        "device": torch.cuda.get_device_name(0), "env": run_env(torch)}), flush=True)
    return 0 if sampled is None or sampled["within_bound"] else 3


def linear_bench(args, torch, dq4, inputs) -> int:
    """Dequantize-plus-linear cells (the issue's public-path controls: the
    forward fallback Y = X W^T and MatMul4Bit grad_A Y = G W) for two weight
    shapes and several token counts m.  Each cell times the whole call
    (fused dequantization + one GEMM), the fused dequantization alone, and the
    unfused three-launch dequantization alone; the GEMM is the same in both
    paths, so the public-path effect of the fusion is
    (t_call - t_fused + t_unfused) / t_call."""
    import itertools
    import math

    import numpy as np

    oracle_cells = []

    def timeit(fn, reps=20):
        warm_up(lambda k: fn(), 0, torch)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps  # us

    cells = []
    for n_out, n_in in ((11008, 4096), (28672, 8192)):
        x = inputs.make_inputs(n_out * n_in, 64, "nf4", 0.03, seed=inputs.SEED_BASE + 6,
                               n_rows=n_out, n_cols=n_in)
        # copies of the quantized weight, cycled so that each call reads it cold
        n_sets = max(1, math.ceil(COLD_PACKED_BYTES / (n_out * n_in // 2)))
        devs = [dq4.to_device(x, "cuda:0") for _ in range(n_sets)]
        turn = itertools.count()

        def dev():
            return devs[next(turn) % n_sets]
        for dt in (torch.float16, torch.bfloat16):
            ws = torch.empty(n_out * n_in, dtype=dt, device="cuda:0")
            sw = torch.empty(dq4.dq4_unfused_workspace_bytes(n_out * n_in, 64) // 4,
                             dtype=torch.float32, device="cuda:0")
            t_fused = timeit(lambda: dq4.dq4_nested_dequant(
                **dev(), offset=float(x.offset), n=n_out * n_in, blocksize=64, out_dtype=dt,
                out=ws))
            t_unfused = timeit(lambda: dq4.dq4_nested_dequant_unfused(
                **dev(), offset=float(x.offset), n=n_out * n_in, blocksize=64, out_dtype=dt,
                out=ws, scale_workspace=sw))
            dt_name = "f16" if dt == torch.float16 else "bf16"
            sample = None
            for op in ("forward", "grad_a"):
                for m in (1, 16, 512, 4096):
                    k = n_in if op == "forward" else n_out
                    xin = torch.randn((m, k), device="cuda:0").to(dt)
                    y = torch.empty((m, n_out if op == "forward" else n_in), dtype=dt,
                                    device="cuda:0")
                    t_call = timeit(lambda: dq4.dq4_dequant_linear(
                        **dev(), offset=float(x.offset), n_out=n_out, n_in=n_in, blocksize=64,
                        x=xin, op=op, y=y, w_workspace=ws))
                    if op == "forward" and m == 16:
                        sample = (xin, y.clone())
                    flops = 2.0 * m * n_out * n_in
                    cell = {"weight": f"{n_out}x{n_in}", "dtype": str(dt).split(".")[-1],
                            "op": op, "m": m, "call_us": round(t_call, 2),
                            "fused_dequant_us": round(t_fused, 2),
                            "unfused_dequant_us": round(t_unfused, 2),
                            "gemm_us": round(max(t_call - t_fused, 0.0), 2),
                            "gemm_TFLOPs": round(flops / max(t_call - t_fused, 1e-3) / 1e6, 2),
                            "gemm_frac_of_matrix_peak": round(
                                flops / max(t_call - t_fused, 1e-3) / 1e6 / MATRIX_PEAK_16BIT, 4),
                            "dequant_frac_of_hbm_peak": round(
                                algorithmic_bytes(n_out * n_in, 64, 2) / (t_fused * 1e-6) / 1e9
                                / HBM_PEAK_GBS, 4),
                            "public_path_speedup": round((t_call - t_fused + t_unfused) / t_call,
                                                         4)}
                    cells.append(cell)
                    print(f"[linear] {cell}", file=sys.stderr, flush=True)
            if not args.no_cpu:
                # the oracle beside it, after this weight's timings: the whole
                # weight, timed, compared bit for bit with the fused
                # dequantization; then the forward m = 16 call against a float64
                # product of the oracle's weight, within the FP32-accumulation
                # and output-rounding bound
                dq4.dq4_nested_dequant(**devs[0], offset=float(x.offset), n=n_out * n_in,
                                       blocksize=64, out_dtype=dt, out=ws)
                w_oracle, t_cpu = oracle_dequant_threaded(x, 0, n_out * n_in, dt_name,
                                                          host_threads())
                oracle_cells.append({
                    "weight": f"{n_out}x{n_in}", "dtype": dt_name, "seconds": round(t_cpu, 4),
                    "cores": host_threads(),
                    "GBps": round(algorithmic_bytes(n_out * n_in, 64, 2) / t_cpu / 1e9, 3),
                    "weight_mismatches": int(np.count_nonzero(device_bits(ws) != w_oracle))})
                xin, y = sample
                wt = torch.from_numpy(w_oracle.view(np.int16)).view(dt).float().numpy()
                w64 = wt.astype(np.float64).reshape(n_out, n_in)
                x64 = xin.float().cpu().numpy().astype(np.float64)
                t0 = time.perf_counter()
                ref = x64 @ w64.T
                t_mm = time.perf_counter() - t0
                s_abs = np.abs(x64) @ np.abs(w64).T
                gk = n_in * 2.0 ** -24 / (1 - n_in * 2.0 ** -24)
                u_out, tiny = ((2.0 ** -11, 2.0 ** -25) if dt == torch.float16
                               else (2.0 ** -8, 2.0 ** -134))
                bound = gk * s_abs + u_out * (np.abs(ref) + gk * s_abs) + tiny
                got = y.float().cpu().numpy().astype(np.float64)
                oracle_cells[-1]["gemm_sample"] = {
                    "op": "forward", "m": 16, "numpy_float64_seconds": round(t_mm, 4),
                    "max_error_over_bound": round(float((np.abs(got - ref) / bound).max()), 4)}
                del w_oracle, wt, w64, x64, ref, s_abs, bound, got
            del ws, sw, sample
        del devs
        torch.cuda.empty_cache()
    sp = [c["public_path_speedup"] for c in cells]
    ok = all(c["weight_mismatches"] == 0 and c["gemm_sample"]["max_error_over_bound"] <= 1.0
             for c in oracle_cells)
    print(json.dumps({
        "metric": "dequantize-plus-linear public-path speedup of the fused dequantization "
                  "(geomean over forward/grad_A cells)",
        "value": round(math.exp(sum(math.log(v) for v in sp) / len(sp)), 4), "unit": "x",
        "higher_is_better": True, "n_gpus": 1, "data": "synthetic", "cells": cells,
        "cpu_baseline": None if args.no_cpu else {
            "kind": "oracle", "cores": host_threads(), "cells": oracle_cells,
            "sample": "per weight and output type: the whole weight through the C oracle "
                      "(compared bit for bit with the fused dequantization), and the "
                      "forward m = 16 product in numpy float64 (the call's result checked "
                      "against it within the accumulation and output-rounding bound)"},
        "device": torch.cuda.get_device_name(0), "env": run_env(torch)}), flush=True)
    return 0 if ok else 3


def int8_prep_bench(args, torch, dq4) -> int:
    """One-launch LLM.int8 correction-operand preparation against the eager
    PyTorch chain it replaces (gather, int8 row-scale dequantization, FP16
    conversion, transposed copy), over the issue's benchmark grid: M in {1, 8,
    64, 512, 2048}, K = N in {3584, 4096, 8192, 14336}, L in {1, 5, 16, 64}."""
    import math

    import numpy as np

    import oracle

    r127 = 7.874015718698502e-3   # float(np.float32(1/127)): the FP32 value nearest 1/127

    def timeit(fn, reps=50):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    g = torch.Generator(device="cuda:0").manual_seed(3)
    cells = []
    dev_ops, dev_cb, roof_ops = [], {}, []
    # --int8-k / --int8-l restrict the grid (the random draws stay those of the
    # whole grid, so a restricted cell has the same operands as in a full run)
    for K in (3584, 4096, 8192, 14336):
        N = K
        CB = torch.randint(-128, 128, (N, K), dtype=torch.int8, device="cuda:0", generator=g)
        SCB = torch.rand(N, device="cuda:0", generator=g) * 10
        if not args.no_cpu:
            dev_cb[K] = (CB, SCB)
        for M in (1, 8, 64, 512, 2048):
            A = torch.randn((M, K), device="cuda:0", generator=g).half()
            for L in (1, 5, 16, 64):
                cols = torch.randperm(K, device="cuda:0", generator=g)[:L].sort().values
                if (args.int8_k and K != args.int8_k) or (args.int8_l and L != args.int8_l):
                    continue
                subA = torch.empty((M, L), dtype=torch.float16, device="cuda:0")
                subB = torch.empty((L, N), dtype=torch.float16, device="cuda:0")
                lib = dq4.library()
                stream = torch.cuda.current_stream().cuda_stream

                def fused():
                    lib.dq4_int8_prep(A.data_ptr(), M, K, CB.data_ptr(), SCB.data_ptr(), N,
                                      cols.data_ptr(), L, subA.data_ptr(), subB.data_ptr(),
                                      stream)

                def eager():
                    ea = A[:, cols].contiguous()
                    eb = (CB[:, cols].contiguous() * SCB.view(-1, 1) * r127).to(
                        torch.float16).t().contiguous()
                    return ea, eb

                t_f = timeit(fused)
                t_e = timeit(eager) if not args.int8_fused_only else float("nan")
                ea, eb = eager()
                fused()
                torch.cuda.synchronize()
                same = bool(torch.equal(ea.view(torch.int16), subA.view(torch.int16)) and
                            torch.equal(eb.view(torch.int16), subB.view(torch.int16)))
                cell = {"M": M, "K": K, "N": N, "L": L, "fused_us": round(t_f, 2),
                        "eager_us": round(t_e, 2), "speedup": round(t_e / t_f, 3),
                        "bit_equal_to_eager": same}
                cells.append(cell)
                roof_ops.append((cell, M, K, N, L, cols))
                if not args.no_cpu:
                    # kept on the device for the oracle pass after every GPU
                    # timing: the timings are host-bound, so no host copies or
                    # CPU work run between them
                    dev_ops.append((cell, K, A, cols, subA.clone(), subB.clone()))
                print(f"[int8] {cells[-1]}", file=sys.stderr, flush=True)
    # the HBM bytes a cell must move: the outputs, and the whole 128-byte lines
    # of A's rows (2-byte elements) and CB's rows (1-byte) that its columns
    # fall in (every K here is a multiple of 64, so rows start on lines), plus
    # SCB and the column list; against the call's time, which at these sizes
    # is mostly the launch
    for cell, M, K, N, L, cols in roof_ops:
        cl = cols.cpu().numpy()
        lines_a = len(set((cl * 2 // 128).tolist()))
        lines_b = len(set((cl // 128).tolist()))
        nbytes = 2 * (M * L + L * N) + 128 * (M * lines_a + N * lines_b) + 4 * N + 8 * L
        cell["roofline"] = {"bound": "hbm", "bytes": nbytes,
                            "GBps": round(nbytes / (cell["fused_us"] * 1e-6) / 1e9, 1),
                            "frac": round(nbytes / (cell["fused_us"] * 1e-6) / 1e9
                                          / HBM_PEAK_GBS, 4)}
    sp = [c["speedup"] for c in cells]
    cpu = None
    if not args.no_cpu:
        # the oracle beside it, on each cell's operands: one thread per call
        def bits(t):
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        host_cb = {K: (CB.cpu().numpy(), SCB.cpu().numpy()) for K, (CB, SCB) in dev_cb.items()}
        for cell, K, A, cols, sub_a, sub_b in dev_ops:
            cb, scb = host_cb[K]
            a_bits, cl, got_a, got_b = bits(A), cols.cpu().numpy(), bits(sub_a), bits(sub_b)
            t0 = time.perf_counter()
            oa, ob = oracle.int8_prep(a_bits, cb, scb, cl)
            cell["oracle_us"] = round((time.perf_counter() - t0) * 1e6, 1)
            cell["bit_equal_to_oracle"] = bool(np.array_equal(oa, got_a) and
                                               np.array_equal(ob, got_b))
        r = [c["oracle_us"] / c["fused_us"] for c in cells]
        cpu = {"kind": "oracle", "cores": 1,
               "oracle_us_range": [min(c["oracle_us"] for c in cells),
                                   max(c["oracle_us"] for c in cells)],
               "gpu_call_speedup_geomean": round(math.exp(sum(map(math.log, r)) / len(r)), 2),
               "all_bit_equal_to_oracle": all(c["bit_equal_to_oracle"] for c in cells),
               "sample": "every cell, one single-threaded oracle call on the same operands"}
    print(json.dumps({
        "metric": "LLM.int8 correction-operand preparation: one kernel vs the eager chain "
                  "(speedup, geomean)",
        "value": round(math.exp(sum(math.log(v) for v in sp) / len(sp)), 3), "unit": "x",
        "higher_is_better": True, "min_speedup": min(sp),
        "median_speedup": sorted(sp)[len(sp) // 2],
        "all_bit_equal": all(c["bit_equal_to_eager"] for c in cells), "cpu_baseline": cpu,
        "roofline_best": max((c["roofline"] for c in cells), key=lambda r: r["frac"]),
        "n_gpus": 1,
        "data": "synthetic", "cells": cells, "device": torch.cuda.get_device_name(0),
        "env": run_env(torch)}),
        flush=True)
    ok = all(c["bit_equal_to_eager"] for c in cells) and (
        cpu is None or cpu["all_bit_equal_to_oracle"])
    return 0 if ok else 3


def configs_bench(args, torch, dq4, inputs) -> int:
    """Every dequantization workload against the HBM roofline, one cell each:
    the 4096^2 FP32 square, the mid-size matrix ({NF4, FP4} x {11008x4096,
    4096x11008} x {FP16, BF16, FP32}), the 28672x8192 headline, the odd-length
    block-size sweep (every block size x NF4/FP4 at one offset: the offset
    changes no instruction or memory access) and the 151936x5376 output head
    as its loop of <= 256 MiB FP32 row windows into one reused buffer.
    Whole-tensor cells cycle enough input/output sets that the packed inputs
    exceed COLD_PACKED_BYTES and time device work from HIP-graph replays; the
    output head's 408 MB packed weight is itself larger than the last-level
    cache, so its window loop runs on one input set, eager and per window."""
    import math

    import numpy as np

    def graph_time(calls, inner):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(inner):
                calls(k)
        warm_up(lambda k: g.replay(), 0, torch)
        samples = []
        for _ in range(max(7, args.batches)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(torch.cuda.current_stream())
            g.replay()
            b.record(torch.cuda.current_stream())
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) * 1e3 / inner)
        del g
        return samples

    def whole_cell(name, x, dt_name, out_shift=0):
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt_name]
        ob = 4 if dt_name == "f32" else 2
        n, bs = x.n, x.blocksize
        alg = algorithmic_bytes(n, bs, ob)
        n_sets = max(2, math.ceil(COLD_PACKED_BYTES / ((n + 1) // 2)))
        # out_shift > 0: the output starts out_shift elements into its buffer,
        # off the 128-byte alignment of the fast path (the general vector path)
        sets = [(dq4.to_device(x, "cuda:0"),
                 torch.empty(n + out_shift, dtype=tdt, device="cuda:0")[out_shift:])
                for _ in range(n_sets)]

        def call(k):
            dev, out = sets[k % n_sets]
            dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=bs,
                                   out_dtype=tdt, out=out)
        for k in range(max(20, n_sets)):
            call(k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream())
        for k in range(n_sets):
            call(k)
        b.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        est_us = max(a.elapsed_time(b) * 1e3 / n_sets, 1.0)
        # whole rounds of the buffer sets, >= 4 ms per replay: shorter batches
        # measure the clock ramp after each synchronization, not the kernel
        inner = n_sets * max(1, math.ceil(4000.0 / (est_us * n_sets)))
        samples = graph_time(call, inner)
        # every set holds the same result; taken before the twin overwrites it
        got = None if args.no_cpu else device_bits(sets[0][1])
        # the memory twin on the same sets where it applies (FP16-sized output,
        # whole 4096-element tiles): the ceiling of the access pattern at this size
        twin_us = None
        if ob == 2 and n % 4096 == 0 and out_shift == 0:
            def twin(k):
                dev, out = sets[k % n_sets]
                dq4.dq4_memory_twin_f16(dev["packed"], n, out=out.view(torch.float16))
            for k in range(n_sets):
                twin(k)
            twin_us = percentile(graph_time(twin, inner), 0.5)
        del sets
        torch.cuda.empty_cache()
        # the oracle beside it: one threaded pass over the whole workload, and
        # every output element compared bit for bit
        oracle_cell = None
        if not args.no_cpu:
            want, t_cpu = oracle_dequant_threaded(x, 0, n, dt_name, host_threads())
            mism = int(np.count_nonzero(got.view(np.uint32 if ob == 4 else np.uint16)
                                        != want.view(np.uint32 if ob == 4 else np.uint16)))
            oracle_cell = {"seconds": round(t_cpu, 4), "cores": host_threads(),
                           "GBps": round(alg / t_cpu / 1e9, 3), "mismatches": mism}
            del want
        del got
        med = percentile(samples, 0.5)
        cell = {"workload": name, "n": n, "blocksize": bs, "format": x.fmt, "out": dt_name,
                "out_shift_elements": out_shift,
                "offset": float(x.offset), "us": round(med, 3),
                "p10_p90": [round(percentile(samples, q), 3) for q in (0.1, 0.9)],
                "algorithmic_bytes": alg, "GBps": round(alg / (med * 1e-6) / 1e9, 1),
                "frac": round(alg / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "ideal_us": round(alg / (HBM_PEAK_GBS * 1e9) * 1e6, 3),
                "buffer_sets": n_sets, "inner": inner,
                "memory_twin_us": None if twin_us is None else round(twin_us, 3),
                "oracle": oracle_cell}
        print(f"[configs] {name}: {med:.2f} us, {cell['GBps']} GB/s ({cell['frac']:.3f})"
              + ("" if twin_us is None else f", memory twin {twin_us:.2f} us")
              + ("" if oracle_cell is None else
                 f"; oracle {oracle_cell['GBps']} GB/s on {oracle_cell['cores']} threads, "
                 f"{oracle_cell['mismatches']} mismatches"),
              file=sys.stderr, flush=True)
        return cell

    cells = []
    wl = inputs.SQUARE_4096_F32
    cells.append(whole_cell(wl.name, wl.inputs(), wl.out_dtype))
    for wl in inputs.mid_matrix_workloads():
        cells.append(whole_cell(wl.name, wl.inputs(), wl.out_dtype))
    wl = inputs.HEADLINE
    x = wl.inputs()
    cells.append(whole_cell(wl.name, x, wl.out_dtype))
    for shift in (1, 8):   # the general vector path: misaligned output
        cells.append(whole_cell(f"{wl.name}_out+{shift}", x, wl.out_dtype, out_shift=shift))
    del x
    for bs in inputs.TAIL_SWEEP_BLOCKSIZES:
        for fmt in ("nf4", "fp4"):
            x = inputs.make_inputs(inputs.TAIL_SWEEP_N, bs, fmt, 0.1, seed=inputs.SEED_BASE + 4)
            cells.append(whole_cell(f"{fmt}_f16_tail_bs{bs}_off+0.1", x, "f16"))

    # the output head: 13 row windows of <= 256 MiB FP32 into one reused buffer
    wl = inputs.OUTPUT_HEAD
    x = wl.inputs()
    dev = dq4.to_device(x, "cuda:0")
    budget = 256 << 20
    windows = dq4.dq4_row_windows(wl.n_rows, wl.n_cols, 4, budget)
    buf = torch.empty(dq4.dq4_rows_per_block(wl.n_cols, 4, budget) * wl.n_cols,
                      dtype=torch.float32, device="cuda:0")

    def window(r0, rows):
        dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=wl.n_rows,
                                    n_cols=wl.n_cols, r0=r0, rows=rows, blocksize=64,
                                    out_dtype=torch.float32, out=buf)
    def loop(k=0):
        for r0, rows in windows:
            window(r0, rows)
    for _ in range(3):
        loop()
    torch.cuda.synchronize()
    graph_loops = graph_time(loop, 6)  # 6 loops of 13 launches per replay (~4 ms)
    stream = torch.cuda.current_stream()
    loops, per_window = [], [[] for _ in windows]
    for _ in range(max(7, args.batches)):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(windows) + 1)]
        evs[0].record(stream)
        for i, (r0, rows) in enumerate(windows):
            window(r0, rows)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        loops.append(evs[0].elapsed_time(evs[-1]) * 1e3)
        for i in range(len(windows)):
            per_window[i].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
    nb = -(-wl.n // 64)
    alg_total = algorithmic_bytes(wl.n, 64, 4)
    win_cells = []
    for (r0, rows), samples in zip(windows, per_window):
        cnt = rows * wl.n_cols
        e0, e1 = r0 * wl.n_cols, (r0 + rows) * wl.n_cols
        # packed bytes, codes and absmax of the blocks and groups the window touches
        b0, b1 = e0 // 64, -(-e1 // 64)
        alg = ((e1 + 1) // 2 - e0 // 2) + (b1 - b0) + 4 * (((b1 - 1) >> 8) - (b0 >> 8) + 1) \
            + 4 * (256 + 16) + 4 * cnt
        med = percentile(samples, 0.5)
        win_cells.append({"r0": r0, "rows": rows, "us": round(med, 3),
                          "GBps": round(alg / (med * 1e-6) / 1e9, 1)})
    med_loop = percentile(graph_loops, 0.5)
    head = {"workload": wl.name, "windows": len(windows), "rows_per_window": windows[0][1],
            "loop_us": round(med_loop, 2),
            "loop_p10_p90": [round(percentile(graph_loops, q), 2) for q in (0.1, 0.9)],
            "eager_loop_us": round(percentile(loops, 0.5), 2),
            "algorithmic_bytes": alg_total, "n_blocks": nb,
            "GBps": round(alg_total / (med_loop * 1e-6) / 1e9, 1),
            "frac": round(alg_total / (med_loop * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "ideal_us": round(alg_total / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
            "per_window": win_cells,
            "timing": "loop_us: 6 loops of the 13 launches replayed as one HIP graph, median "
                      "of >= 7 replays; eager_loop_us and per_window: eager launches with one HIP "
                      "event after each window"}
    if not args.no_cpu:
        # the oracle over the whole head, timed; the reused buffer still holds
        # the last window, compared bit for bit with the oracle's rows
        want, t_cpu = oracle_dequant_threaded(x, 0, wl.n, "f32", host_threads())
        r0, rows = windows[-1]
        got = device_bits(buf[: rows * wl.n_cols])
        mism = int(np.count_nonzero(
            got.view(np.uint32) != want[r0 * wl.n_cols:(r0 + rows) * wl.n_cols].view(np.uint32)))
        head["oracle"] = {"seconds": round(t_cpu, 4), "cores": host_threads(),
                          "GBps": round(alg_total / t_cpu / 1e9, 3),
                          "compared": f"last window, rows {r0}..{r0 + rows - 1}",
                          "mismatches": mism}
        del want, got
    print(f"[configs] {wl.name}: {len(windows)} windows in {med_loop:.1f} us, "
          f"{head['GBps']} GB/s ({head['frac']:.3f})"
          + ("" if "oracle" not in head else
             f"; oracle {head['oracle']['GBps']} GB/s, {head['oracle']['mismatches']} mismatches"),
          file=sys.stderr, flush=True)
    del buf, dev
    print(json.dumps({
        "metric": "dequantized GB/s per workload (fraction of HBM peak)",
        "unit": "GB/s", "higher_is_better": True, "n_gpus": 1, "data": "synthetic",
        "timing": "device time per call from HIP-graph replays over cycled cold input sets, "
                  "median of >= 7 batches",
        "cells": cells, "output_head": head, "device": torch.cuda.get_device_name(0),
        "env": run_env(torch)}),
        flush=True)
    checked = [c["oracle"] for c in cells if c["oracle"]] + (
        [head["oracle"]] if "oracle" in head else [])
    return 0 if all(o["mismatches"] == 0 for o in checked) else 3


def launch_trace(args, torch, dq4, inputs) -> int:
    """Three phases for a launch/allocation trace (rocprofv3 --kernel-trace
    --hip-trace --memory-allocation-trace): 10 fused calls into the caller's
    output, 10 unfused calls with the caller's scale workspace, and 10
    unfused calls where the binding allocates that workspace (torch's cache
    emptied after each call).  Everything else is allocated up front; a
    one-element torch add and a synchronization mark each phase boundary."""
    n = 4096 * 4096
    x = inputs.make_inputs(n, 64, "nf4", 0.03, seed=inputs.SEED_BASE + 1, n_rows=4096,
                           n_cols=4096)
    dev = dq4.to_device(x, "cuda:0")
    out = torch.empty(n, dtype=torch.float16, device="cuda:0")
    ws = torch.empty(dq4.dq4_unfused_workspace_bytes(n, 64) // 4, dtype=torch.float32,
                     device="cuda:0")
    marker = torch.zeros(1, device="cuda:0")
    kw = dict(offset=float(x.offset), n=n, blocksize=64, out_dtype=torch.float16, out=out)
    torch.cuda.synchronize()

    def mark():
        marker.add_(1.0)
        torch.cuda.synchronize()
    mark()
    for _ in range(10):
        dq4.dq4_nested_dequant(**dev, **kw)
    mark()
    for _ in range(10):
        dq4.dq4_nested_dequant_unfused(**dev, **kw, scale_workspace=ws)
    mark()
    torch.cuda.empty_cache()
    for _ in range(10):
        dq4.dq4_nested_dequant_unfused(**dev, **kw)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    mark()
    print(json.dumps({"launch_trace": "phases done", "n": n}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=700, help="timed steps (then sampled again in 7 batches)")
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (>= 20; the default lets clocks settle)")
    ap.add_argument("--rotate", type=int, default=6,
                    help="independent buffer sets cycled (6 x 117 MB of packed input is "
                         "2.7x the 256 MB last-level cache, so every read is cold)")
    ap.add_argument("--batches", type=int, default=7)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline (whole-tensor passes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline and parity")
    ap.add_argument("--compare-unfused", action="store_true",
                    help="instead of the benchmark, time the fused kernel against the unfused "
                         "three-launch sequence over the primary standalone matrix")
    ap.add_argument("--out-prod", action="store_true",
                    help="instead of the benchmark, time the row-blocked out_prod of the "
                         "151936x5376 output head (FP32 GEMM per window)")
    ap.add_argument("--out-prod-m", type=int, default=512,
                    help="columns of src1 (tokens) for --out-prod")
    ap.add_argument("--out-prod-transposed", action="store_true",
                    help="--out-prod: src1 stored transposed (m x n_rows) for both routes")
    ap.add_argument("--linear", action="store_true",
                    help="instead of the benchmark, time dequantize-plus-linear forward and "
                         "grad_A cells")
    ap.add_argument("--int8-prep", action="store_true",
                    help="instead of the benchmark, time the LLM.int8 correction-operand "
                         "preparation against the eager chain")
    ap.add_argument("--int8-k", type=int, default=0,
                    help="--int8-prep: only the cells with this K (= N)")
    ap.add_argument("--int8-l", type=int, default=0,
                    help="--int8-prep: only the cells with this many outlier columns")
    ap.add_argument("--int8-fused-only", action="store_true",
                    help="--int8-prep: time the one-kernel call only (for counter runs)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the benchmark, time every dequantization workload (square, "
                         "mid matrix, headline, block-size sweep, output-head window loop) "
                         "against the HBM roofline")
    ap.add_argument("--launch-trace", action="store_true",
                    help="instead of the benchmark, run the fused and unfused calls in marked "
                         "phases for a rocprofv3 launch and allocation trace")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, time a plain device-to-device copy of MIB "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for {args.gpus}); the "
              "dequantization shards without any exchange, so there is no multi-GPU step to time.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_wise_bit_amd as dq4
    from block_wise_bit_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        return copy_calibration(args, torch)
    dq4.library()  # fail loudly if the HIP library is missing
    if args.compare_unfused:
        return compare_unfused(args, torch, dq4, inputs)
    if args.out_prod:
        return out_prod_bench(args, torch, dq4, inputs)
    if args.linear:
        return linear_bench(args, torch, dq4, inputs)
    if args.int8_prep:
        return int8_prep_bench(args, torch, dq4)
    if args.configs:
        return configs_bench(args, torch, dq4, inputs)
    if args.launch_trace:
        return launch_trace(args, torch, dq4, inputs)

    wl = inputs.HEADLINE
    n, bs = wl.n, wl.blocksize
    out_bytes = 2
    alg_bytes = algorithmic_bytes(n, bs, out_bytes)
    print(f"[bench] workload {wl.name}: n={n} bs={bs} algorithmic bytes/step={alg_bytes}",
          file=sys.stderr, flush=True)

    x = wl.inputs()
    sets = []
    for r in range(max(1, args.rotate)):
        dev = dq4.to_device(x, "cuda:0")
        out = torch.empty(n, dtype=torch.float16, device="cuda:0")
        sets.append((dev, out))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    offset = float(x.offset)

    # every buffer set goes through the checked torch wrapper once, then the
    # steps call the C entry point with those same, already checked arguments:
    # the wrapper's Python checks cost tens of microseconds per call, which
    # would leave the stream idle between launches
    for dev, out in sets:
        dq4.dq4_nested_dequant(**dev, offset=offset, n=n, blocksize=bs, out_dtype=torch.float16,
                               out=out, stream=stream)
    step = raw_dequant_steps(dq4, sets, offset, n, bs, dq4.DQ4_F16, stream)

    K = args.steps
    nbatch = max(1, min(args.batches, K))
    per = [K // nbatch + (1 if i < K % nbatch else 0) for i in range(nbatch)]

    warm = warm_up(step, args.warmup, torch)
    print(f"[bench] {warm} warmup steps done ({args.warmup} asked for)", file=sys.stderr,
          flush=True)

    # timed region: K steps with one event pair around all of them on the
    # launch stream, and the wall clock around the region.  (An event recorded
    # between two launches holds the next launch back until the timestamp is
    # written, so the per-batch events stay out of this region.)
    kernel_us, wall = timed_region(step, K, stream, torch)
    ms_per_step = wall * 1e3 / K
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kernel_us * 1e-6) / 1e9
    print(f"[bench] {K} timed steps: {ms_per_step * 1e3:.2f} us/step wall, "
          f"{kernel_us:.2f} us/launch (events)", file=sys.stderr, flush=True)

    # the spread: the same K steps again, right after the timed region, in
    # `batches` batches with an event pair each
    batch_us = timed_batches(step, per, stream, torch, first=K)
    # the timed region's last output, for the parity check: the batches wrote
    # the same bits into it again (the call is deterministic), and the copy
    # waits until now so that the GPU does not idle before the batches
    last_out = sets[(K - 1) % len(sets)][1].cpu()

    # the memory twin, timed the same way on the same buffer sets: the same
    # tiles, loads and stores with no arithmetic -- the ceiling of this access
    # pattern on this GPU
    twin_bytes = (n + 1) // 2 + 2 * n

    for dev, out in sets:
        dq4.dq4_memory_twin_f16(dev["packed"], n, out=out, stream=stream)
    twin = raw_twin_steps(dq4, sets, n, stream)
    warm_up(twin, args.warmup, torch)
    twin_us, _ = timed_region(twin, K, stream, torch)
    print(f"[bench] memory twin: {twin_us:.2f} us/launch (events)", file=sys.stderr, flush=True)

    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_launches": warm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_rows": wl.n_rows, "n_cols": wl.n_cols,
                   "format": wl.fmt, "out_dtype": "f16", "blocksize": bs,
                   "nested_blocksize": 256, "offset": wl.offset, "seed": wl.seed,
                   "buffer_sets": len(sets), "input_digest": x.digest()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "elements_per_s": round(n / (kernel_us * 1e-6), 1),
        "kernel_us": {"mean": round(kernel_us, 3),
                      "batches_after": [round(b, 3) for b in batch_us],
                      "median": round(percentile(batch_us, 0.5), 3),
                      "p10": round(percentile(batch_us, 0.1), 3),
                      "p90": round(percentile(batch_us, 0.9), 3)},
        "kernel_isa_sha256_16": kernel_digest(),
        "attainable": {"kernel": "dq4_memory_twin_kernel: the same tiles, tile order, loads and "
                                 "stores, no arithmetic and no metadata",
                       "us": round(twin_us, 3), "bytes_per_launch": twin_bytes,
                       "GBps": round(twin_bytes / (twin_us * 1e-6) / 1e9, 2),
                       "frac_of_peak": round(twin_bytes / (twin_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                             4),
                       "dequant_over_twin_time": round(kernel_us / twin_us, 4)},
        "device": torch.cuda.get_device_name(0), "env": run_env(torch),
        "cpu_baseline": None,
        "parity": None,
    }

    if not args.no_cpu:
        got = last_out.view(torch.int16).numpy().view(np.uint16)

        def timed_passes(threads):
            passes, t_cpu, want = 0, 0.0, None
            while passes < 3 and (passes == 0 or t_cpu < args.cpu_seconds):
                want, dt = oracle_dequant_threaded(x, 0, n, "f16", threads)
                t_cpu += dt
                passes += 1
                print(f"[bench] oracle on {threads} thread(s), pass {passes}: {t_cpu:.2f} s so "
                      f"far", file=sys.stderr, flush=True)
            return passes, t_cpu, want

        threads = host_threads()
        passes, t_cpu, want = timed_passes(threads)
        passes1, t_cpu1, want1 = timed_passes(1)
        mismatches = int(np.count_nonzero(got != want))
        host = (f"host {platform.processor() or platform.machine()} with {os.cpu_count()} "
                f"logical cpus")
        result["cpu_baseline"] = {
            "value": round(alg_bytes * passes / t_cpu / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"whole {wl.n_rows}x{wl.n_cols} tensor, {passes} pass(es) on {threads} "
                      f"threads over disjoint element ranges, {t_cpu:.2f} s; {host}",
            "elements_per_s": round(n * passes / t_cpu, 1),
            "single_core": {"value": round(alg_bytes * passes1 / t_cpu1 / 1e9, 4),
                            "unit": "GB/s", "cores": 1,
                            "sample": f"whole tensor, {passes1} single-threaded pass(es), "
                                      f"{t_cpu1:.2f} s",
                            "elements_per_s": round(n * passes1 / t_cpu1, 1)}}
        result["parity"] = {"compared_elements": n, "mismatches": mismatches,
                            "bit_exact": mismatches == 0,
                            "threaded_oracle_equals_single_threaded":
                                bool(np.array_equal(want, want1))}

    print(json.dumps(result), flush=True)
    if result["parity"] is not None and not result["parity"]["bit_exact"]:
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
