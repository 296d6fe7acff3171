"""Throughput of the fp32 GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one C = A x B call through the C ABI (gemm_f32, the default
kernel) on seeded synthetic operands already resident in HBM.  The step runs
untimed for --settle-s seconds (default 2 for this headline line, 0.3 for the
other modes: the clock ramps up after the idle spell of input generation),
then W untimed steps, then exactly K timed steps between two device
synchronisations.  One
JSON line is printed with the metric (TFLOP/s = 2MNK per step / seconds),
the roofline of the kernel (algorithmic FLOP per launch over the average
launch time from HIP events on the launch stream, against the chip's
published fp32 peak, plus the HBM bytes per launch from hardware counters
when those were taken on the current kernel source), and a CPU baseline:
the oracle timed on this host's cores on a bounded band of output rows.

Extra modes (used for counter runs under rocprofv3):
    --ladder            time every rung and diagnostic variant instead
    --copy-probe-mib N  first run one device-to-device copy of N MiB, the
                        reference for scaling HBM byte counters
    --no-cpu-baseline   skip the oracle timing
    --row transpose     time transpose_f32 on the workload's A matrix instead
                        (metric GB/s moved, bound HBM); the launches cycle
                        through --rotate copies (default 4: a cold cache),
                        and the same matrix repeated is reported beside it
    --variants LIST     with --ladder: only these variant numbers
    --view-offset N     floats between each allocation and its matrix view
                        (default: the workload's own)
    --row reduce        time reduce_sum_f32 on --n uniform[-1,1) values
                        (default 2^28; metric GB/s read, bound HBM)
    --row mixed         time gemm_mixed on the workload rounded to --format
                        (bf16 or f16; binary32 result; metric TFLOP/s against
                        the 16-bit matrix peak); with --op, gemm_mixed_op
    --op XY             time gemm_f32_op with op(A) = X, op(B) = Y (N or T):
                        the transposed factor is stored transposed, with a
                        compact leading dimension
    --all-workloads     gemm_f32 at each of the five workloads (the padded
                        rect workload also with aligned views, offset 0): one
                        JSON line per run with the median and best launch time
                        (HIP events around every launch), then the oracle's
                        time on this host (see bench_all_workloads)
    --copy-rate         bytes per clock per CU that 1 KB wave loads bring from
                        an L2-resident buffer into LDS and into registers
    --lds-probe         one wave reading LDS at chosen offsets, one launch per
                        case (which lanes one read cycle serves, from the
                        bank-conflict counter of each dispatch)
    --valu-probe        the issue rate of non-packed v_fmac_f32 on the vector
                        ALU in three operand forms, with the measured clock
                        (the register-blocked rung's ceiling)
    --shape-sweep       the tile choice on 37 shapes (512^3 .. 8192^3,
                        rectangular and awkward ones): TFLOP/s of the default
                        configuration, of every candidate configuration and
                        of torch.matmul (hipBLASLt, for context), one JSON
                        line per shape (see bench_shape_sweep); with --row
                        mixed, of gemm_mixed in --format; --shapes MxNxK,...
                        runs those shapes only
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3        # MI355X published dense fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0
PEAK_16BIT_TFLOPS = 2500.0      # MI355X published dense bf16 / fp16 matrix peak
DEFAULT_WORKLOAD = "square8192"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mfma_square8192_hbm_traffic.txt")
KERNEL_SOURCES = ["shared_memory_tiled_amd/csrc/mfma_sched.hip",
                  "shared_memory_tiled_amd/csrc/gemm_internal.h"]


def source_code(text: str) -> str:
    """The code of a C++ source without its comments and with whitespace
    runs collapsed (the kernel sources hold no string literals with // or
    /*), so that an edit of a comment leaves the digest unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(source_code(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing, for another workload, or taken on different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [l for l in f if l.startswith("TRAFFIC_JSON ")]
        rec = json.loads(lines[-1][len("TRAFFIC_JSON "):])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(A, B, w, op_a="N", op_b="N", budget_s: float = 12.0):
    """The oracle as it is, on all host cores, over a band of output rows."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    rows = min(cores, w.M)                  # one row per thread to size the sample
    t0 = time.perf_counter()
    oracle.gemm(A.view, B.view, threads=cores, rows=(0, rows), op_a=op_a, op_b=op_b)
    probe = time.perf_counter() - t0
    rows = max(rows, min(w.M, int(rows * budget_s / max(probe, 1e-3))))
    rows -= rows % cores if rows > cores else 0
    t0 = time.perf_counter()
    oracle.gemm(A.view, B.view, threads=cores, rows=(0, rows), op_a=op_a, op_b=op_b)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * w.N * w.K
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} product "
                      f"({rows * w.N} outputs, {flop:.3e} FLOP) in {dt:.2f} s, binary64 "
                      f"triple loop, {cores} threads"}


# Untimed run of the step, in seconds, before its warm-up steps.  After an
# idle spell (host-side input generation) the GPU's clock ramps back up over
# some tens of milliseconds: measured, a 4096^3 product's launches speed up
# by about 20 % over their first 25 ms, and a step of a fraction of a
# millisecond would otherwise be timed entirely on that ramp.
SETTLE_S = 0.3
# The headline line settles longer: its timed region is short (tens of
# milliseconds), and a longer untimed stretch of the same step keeps the GPU
# visibly busy to outside utilisation samplers as well.
HEADLINE_SETTLE_S = 2.0


def settle(fn, seconds=None) -> int:
    """Runs fn untimed for `seconds` (default SETTLE_S) of wall time; returns
    the number of calls."""
    import torch
    seconds = SETTLE_S if seconds is None else seconds
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def graph_ms_per_launch(fn, launches: int, replays: int = 5):
    """Per-launch time of `fn` when `launches` calls of it are captured in
    one HIP graph and the graph is replayed: the launches then run back to
    back on the GPU, with no host in between.  A product of a few
    microseconds takes less time on the GPU than one call through Python
    takes on the host, so timing eager calls measures the host.  The graph is
    replayed untimed for 0.3 s first (steady clock), then `replays` times
    between HIP events; returns the per-launch times of those replays, in
    milliseconds.  The library enqueues only kernel launches (no memory
    operations), which capture as kernel nodes."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    torch.cuda.synchronize()
    settle(g.replay)
    out = []
    stream = torch.cuda.current_stream()
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / launches)
    del g
    return out


def _timed(fn, steps, warmup):
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1) / steps


def bench_reduce(args) -> int:
    """reduce_sum_f32 over n uniform[-1,1) floats resident in HBM; bytes read
    = 4 n per launch (the partials are a few KB)."""
    import numpy as np
    import torch

    from shared_memory_tiled_amd import binding, inputs

    n = args.n
    x_host = inputs.random_matrix(inputs.rng(100, 0), 1, n, "uniform").reshape(-1)
    x = torch.from_numpy(x_host).cuda()
    out = torch.empty(1, device="cuda")
    read = 4.0 * n

    def make(v):
        vv = binding.REDUCE_DEFAULT if v is None else v
        wsb = binding.reduce_sum_f32_workspace_size(vv, n)
        ws = torch.empty(max(wsb // 4, 1), device="cuda")
        if v is None:
            return lambda: binding.reduce_sum_f32(n, x, out, ws, wsb)
        return lambda: binding.reduce_sum_f32_variant(v, n, x, out, ws, wsb)

    if args.ladder:
        for v in range(binding.reduce_sum_f32_num_variants()):
            _, ms = _timed(make(v), args.steps, 1)
            print(json.dumps({"row": "reduce", "variant": v, "name": binding.reduce_sum_f32_variant_name(v),
                              "n": n, "ms_per_launch": round(ms, 4), "GB_per_s": round(read / ms / 1e6, 1)}),
                  flush=True)
        return 0
    wall, ms = _timed(make(args.variant), args.steps, args.warmup)
    _, torch_ms = _timed(lambda: torch.sum(x), args.steps, args.warmup)
    achieved = read / (ms * 1e-3) / 1e9
    line = {
        "metric": "fp32 sum reduction GB/s (bytes read) on MI355X",
        "value": round(read * args.steps / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"sum of {n} uniform[-1,1) floats", "n": n,
                   "kernel": binding.reduce_sum_f32_variant_name(binding.REDUCE_DEFAULT if args.variant is None
                                                                 else args.variant),
                   "torch_sum_same_data_GB_per_s": round(read / (torch_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.reduce_sum(x_host)
            reps += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(read * reps / dt / 1e9, 2), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "sample": f"{reps} full sums of {n} values in {dt:.2f} s, one thread"}
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline16(fmt, A, B, w, budget_s: float = 10.0, op_a="N", op_b="N"):
    """The 16-bit oracle as it is, on all host cores, over a band of rows."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    rows = min(cores, w.M)
    t0 = time.perf_counter()
    oracle.gemm16(fmt, A.view, B.view, threads=cores, rows=(0, rows), op_a=op_a, op_b=op_b)
    probe = time.perf_counter() - t0
    rows = max(rows, min(w.M, int(rows * budget_s / max(probe, 1e-3))))
    rows -= rows % cores if rows > cores else 0
    t0 = time.perf_counter()
    oracle.gemm16(fmt, A.view, B.view, threads=cores, rows=(0, rows), op_a=op_a, op_b=op_b)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * w.N * w.K
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} {fmt} product "
                      f"({rows * w.N} outputs, {flop:.3e} FLOP) in {dt:.2f} s, binary64 "
                      f"triple loop, {cores} threads"}


def bench_mixed(args, w) -> int:
    """gemm_mixed on the workload's data rounded to 16 bits (bf16 or f16),
    binary32 result; 2 M N K FLOP per launch against the 16-bit matrix peak."""
    import numpy as np
    import torch

    from shared_memory_tiled_amd import binding, inputs

    fmt = args.format
    op_a, op_b = args.op[0], args.op[1]
    A, B, _, _ = inputs.operands16(w, fmt)
    lda, ldb = w.lda, w.ldb
    if args.op != "NN":     # the transposed factor is stored transposed (compact rows)
        if op_a == "T":
            A = inputs.padded16(np.ascontiguousarray(A.view.T), w.M, w.offset, fmt)
            lda = w.M
        if op_b == "T":
            B = inputs.padded16(np.ascontiguousarray(B.view.T), w.K, w.offset, fmt)
            ldb = w.K
    dev = torch.device("cuda:0")
    a = torch.from_numpy(A.buf.view(np.int16)).to(dev)
    b = torch.from_numpy(B.buf.view(np.int16)).to(dev)
    c = torch.empty(w.offset + w.M * w.ldc + 64, dtype=torch.float32, device=dev)
    call_args = (fmt, w.M, w.N, w.K, a.data_ptr() + 2 * w.offset, lda, b.data_ptr() + 2 * w.offset,
                 ldb, c.data_ptr() + 4 * w.offset, w.ldc)
    flop = 2.0 * w.M * w.N * w.K

    def make(v):
        if args.op != "NN":
            return lambda: binding.gemm_mixed_op(op_a, op_b, *call_args)
        if v is None:
            return lambda: binding.gemm_mixed(*call_args)
        return lambda: binding.gemm_mixed_variant(v, *call_args)

    if args.ladder:
        for v in range(binding.gemm_mixed_num_variants()):
            _, ms = _timed(make(v), args.steps, 2)
            print(json.dumps({"row": "mixed", "format": fmt, "variant": v,
                              "name": binding.gemm_mixed_variant_name(v), "workload": w.name,
                              "ms_per_launch": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                              "frac_of_peak": round(flop / ms / 1e9 / PEAK_16BIT_TFLOPS, 4)}), flush=True)
        return 0
    wall, ms = _timed(make(args.variant), args.steps, args.warmup)
    achieved = flop / (ms * 1e-3) / 1e12
    picked = binding.gemm_mixed_default_variant(w.M, w.N, w.K)     # the configuration gemm_mixed runs
    config = {"workload": f"{w.name} rounded to {fmt}", "M": w.M, "N": w.N, "K": w.K, "lda": lda,
              "ldb": ldb, "ldc": w.ldc, "view_offset_elements": w.offset, "values": w.dist,
              "format": fmt, "result": "f32", "op": args.op,
              "kernel": (f"gemm_mixed_op({op_a},{op_b})" if args.op != "NN" else
                         binding.gemm_mixed_variant_name(picked if args.variant is None else args.variant))}
    if args.op == "NN" and w.offset == 0 and w.lda == w.K and w.ldb == w.N:
        dt = torch.bfloat16 if fmt == "bf16" else torch.float16
        at = a[:w.M * w.K].view(dt).view(w.M, w.K)
        bt = b[:w.K * w.N].view(dt).view(w.K, w.N)
        _, tms = _timed(lambda: torch.matmul(at, bt), args.steps, args.warmup)
        config["torch_matmul_same_inputs_16bit_out_TFLOPs"] = round(flop / tms / 1e9, 1)
    line = {
        "metric": f"{fmt} x {fmt} -> f32 GEMM TFLOP/s on MI355X",
        "value": round(flop * args.steps / wall / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": fmt,
        "data": "synthetic", "config": config,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_16BIT_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_16BIT_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline16(fmt, A, B, w, op_a=op_a, op_b=op_b)
    print(json.dumps(line), flush=True)
    return 0


def bench_transpose(args, w) -> int:
    """transpose_f32 of the workload's A matrix (M x K, leading dimension lda)
    into an M-column output; bytes moved = 2 x 4 M K per launch.

    Cold: the launches cycle through --rotate distinct input/output pairs
    (copies of the same matrix), so at square8192 (256 MiB in, 256 MiB out)
    with the default 4 pairs each launch reads a matrix that 1.5 GiB of
    other traffic has passed since it was last touched -- far more than the
    256 MB last-level cache holds -- and the rate is an HBM rate.  The same
    matrix transposed over and over (one pair) is also timed and reported as
    cache-assisted: its input fits the last-level cache."""
    import torch

    from shared_memory_tiled_amd import binding, inputs

    A, _ = inputs.operands(w)
    dev = torch.device("cuda:0")
    rotate = max(1, args.rotate)
    a0 = torch.from_numpy(A.buf).to(dev)
    ins = [a0] + [a0.clone() for _ in range(rotate - 1)]
    outs = [torch.empty(w.K * w.M + 64, dtype=torch.float32, device=dev) for _ in range(rotate)]
    moved = 2.0 * 4 * w.M * w.K
    state = {"variant": args.variant, "i": 0}

    def call(x, y):
        targs = (w.M, w.K, x.data_ptr() + 4 * w.offset, w.lda, y.data_ptr(), w.M)
        if state["variant"] is None:
            binding.transpose_f32(*targs)
        else:
            binding.transpose_f32_variant(state["variant"], *targs)

    def one():                        # cold: the next pair in turn
        i = state["i"] % rotate
        state["i"] += 1
        call(ins[i], outs[i])

    def same():                       # cache-assisted: always the first pair
        call(ins[0], outs[0])

    if args.ladder:
        for v in range(binding.transpose_f32_num_variants()):
            state["variant"] = v
            _, ms = _timed(one, args.steps, 1)
            print(json.dumps({"row": "transpose", "variant": v, "name": binding.transpose_f32_variant_name(v),
                              "workload": w.name, "rotate": rotate, "ms_per_launch": round(ms, 4),
                              "GB_per_s": round(moved / ms / 1e6, 1)}), flush=True)
        return 0
    wall, ms = _timed(one, args.steps, args.warmup)
    _, same_ms = _timed(same, args.steps, args.warmup)
    # the same bytes through a plain device copy, for reference (rotated too)
    srcs = [x[w.offset:w.offset + w.M * w.lda] for x in ins]
    dsts = [torch.empty_like(srcs[0]) for _ in range(rotate)]
    cstate = {"i": 0}

    def copy_one():
        i = cstate["i"] % rotate
        cstate["i"] += 1
        dsts[i].copy_(srcs[i])

    _, copy_ms = _timed(copy_one, args.steps, args.warmup)
    achieved = moved / (ms * 1e-3) / 1e9
    copy_bytes = 2.0 * 4 * w.M * w.lda
    line = {
        "metric": "fp32 shared-tile transpose GB/s (bytes read + written) on MI355X",
        "value": round(moved * args.steps / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} A matrix", "rows": w.M, "cols": w.K, "ld_in": w.lda,
                   "ld_out": w.M, "view_offset_floats": w.offset,
                   "rotate": rotate,
                   "cache": ("cold: each launch's input last touched "
                             f"{(rotate - 1) * 2 * 4 * w.M * w.K / 2**20:.0f} MiB of traffic earlier"
                             if rotate > 1 else "same matrix every launch"),
                   "kernel": ("auto: " + binding.transpose_f32_variant_name(
                       binding.transpose_f32_default_variant(w.M, w.K, w.lda, w.M)))
                   if args.variant is None else binding.transpose_f32_variant_name(args.variant),
                   "cache_assisted_same_matrix_GB_per_s": round(moved / (same_ms * 1e-3) / 1e9, 1),
                   "device_copy_same_bytes_rotated_GB_per_s": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle
        t0 = time.perf_counter()
        reps = 0
        buf = np.zeros((w.K, w.M), dtype=np.float32)
        while time.perf_counter() - t0 < 10.0:
            oracle.transpose_into(A.view, buf)
            reps += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(moved * reps / dt / 1e9, 2), "unit": "GB/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{reps} full {w.M}x{w.K} transposes in {dt:.2f} s, one thread"}
    print(json.dumps(line), flush=True)
    return 0


# Timed launches per workload: many for the microsecond-scale small products
# (100 per timed window, so that the event between windows weighs little),
# fewer for the large ones.
WORKLOAD_LAUNCHES = {"square256": 1000, "square1000": 1000, "square4096": 20,
                     "rect8192x4096x2048_padded": 20, "square8192": 10}


SWEEP_SHAPES = ([(n, n, n) for n in (512, 768, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 4352, 4608, 5120,
                                      6144, 7168, 8192)] +
                [(4100, 4100, 4096), (4000, 5000, 4096), (6000, 6000, 6000), (8200, 8200, 4096),
                 (8192, 4096, 2048), (2048, 8192, 4096), (16384, 1024, 4096), (1024, 16384, 2048),
                 (5000, 3000, 2000), (3000, 7000, 1024), (1000, 2000, 500), (2048, 2048, 256),
                 (4096, 4096, 256), (1024, 1024, 4096), (1000, 1000, 1000), (3000, 3000, 384),
                 (8192, 8192, 8100), (4096, 4096, 4100), (2304, 2304, 2304), (2816, 2816, 2816),
                 (2048, 4096, 1024), (2048, 3072, 512)])
SWEEP_CANDIDATES = ["mfma64x64_bk32_w2x2_k4", "mfma64x64_bk16_w2x2_k4", "mfma64x64_bk32_w1x1_k4_sched",
                    "mfma128x128_bk16_w2x2",
                    "mfma128x128_bk32_w2x2_sched", "mfma256x256_bk32_w2x4_direct",
                    "mfma256x256_bk32_w2x2_sched", "mfma96x96_bk16_w1x1_k4_sched", "mfma64x64_bk32_w2x2_sched"]


MIXED_SWEEP_CANDIDATES = ["mixed64x64_bk64_w1x2", "mixed64x64_bk32_w4_ksplit", "mixed128x128_bk64_w2x2_directAB",
                          "mixed256x256_bk64_w2x4_directAB", "mixed256x256_bk64_w4_sched",
                          "mixed256x256_bk64_w4_wide", "mixed256x256_bk32_w4_wide4stage", "mixed128x128_bk32_w4_ksplit",
                          "mixed192x192_bk64_w4_wide", "mixed256x256_rowsplit", "mixed160x160_bk64_w4_wide"]


def bench_shape_sweep(args) -> int:
    """For each shape (uniform[-1,1) operands, compact leading dimensions):
    the configuration gemm_f32 picks and the TFLOP/s of every candidate
    configuration through gemm_f32_variant, each as 10 launches captured in
    a HIP graph, replayed untimed for 0.3 s, then timed over 3 replays (the
    median per launch; see graph_ms_per_launch), plus
    torch.matmul on the same operands (fp32, TF32 off) for context.  With
    --row mixed the same for gemm_mixed on operands rounded to --format
    (binary32 result), against torch.matmul in that format (16-bit result)."""
    import torch

    from shared_memory_tiled_amd import binding

    torch.backends.cuda.matmul.allow_tf32 = False
    mixed = args.row == "mixed"
    if mixed:
        dtype = torch.bfloat16 if args.format == "bf16" else torch.float16
        number = {binding.gemm_mixed_variant_name(v): v for v in range(binding.gemm_mixed_num_variants())}
        candidates = MIXED_SWEEP_CANDIDATES
        default_name = lambda M, N, K: binding.gemm_mixed_variant_name(binding.gemm_mixed_default_variant(M, N, K))
        run = lambda X, Y, out, v=None: binding.gemm16(X, Y, out, variant=v)
        context = lambda X, Y, out: torch.matmul(X, Y)
    else:
        dtype = torch.float32
        number = {binding.gemm_f32_variant_name(binding.DIAGNOSTIC_BASE + d): binding.DIAGNOSTIC_BASE + d
                  for d in range(binding.gemm_f32_num_diagnostic_variants())}
        candidates = SWEEP_CANDIDATES
        default_name = lambda M, N, K: binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(M, N, K))
        run = lambda X, Y, out, v=None: binding.gemm(X, Y, out, variant=v)
        context = lambda X, Y, out: torch.matmul(X, Y, out=out)

    def tflops(fn, flop, reps=10):
        import statistics
        return flop / statistics.median(graph_ms_per_launch(fn, reps, replays=3)) / 1e9

    gen = torch.Generator(device="cuda").manual_seed(20261202)
    shapes = SWEEP_SHAPES
    if args.shapes:                     # e.g. 3072x3072x3072,4352x4352x4352
        shapes = [tuple(int(x) for x in sh.split("x")) for sh in args.shapes.split(",")]
    for (M, N, K) in shapes:
        X = (torch.rand((M, K), device="cuda", generator=gen) * 2 - 1).to(dtype)
        Y = (torch.rand((K, N), device="cuda", generator=gen) * 2 - 1).to(dtype)
        out = torch.empty((M, N), device="cuda")
        flop = 2.0 * M * N * K
        res = {c: round(tflops(lambda: run(X, Y, out, number[c]), flop), 1) for c in candidates}
        best = max(res, key=res.get)
        line = {"M": M, "N": N, "K": K, "dtype": str(dtype).replace("torch.", ""), "default": default_name(M, N, K),
                "default_tflops": round(tflops(lambda: run(X, Y, out), flop), 1),
                "best": best, "best_tflops": res[best], "candidates_tflops": res,
                "torch_matmul_tflops": round(tflops(lambda: context(X, Y, out), flop), 1)}
        line["default_over_best"] = round(line["default_tflops"] / res[best], 3)
        print(json.dumps(line), flush=True)
        del X, Y, out
    return 0


def bench_valu_probe(args) -> int:
    """The vector-ALU issue rate of the register-blocked rung's instruction
    (non-packed v_fmac_f32), from the library's measurement helper: each
    operand form at 4 and 8 waves per SIMD, three runs each, with the clock
    the loop ran at (shader clock counter against the 100 MHz counter) and
    the wave64 FMAs issued per SIMD per clock at that clock."""
    import torch

    from shared_memory_tiled_amd import binding

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    forms = {0: "scalar-register operand", 1: "vector registers", 2: "8x8 outer product"}
    for form, what in forms.items():
        for wps in (4, 8):
            blocks = cus * wps                    # 4 waves per block: one per SIMD
            waves = blocks * 4
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            stamps = torch.zeros(waves * 4, dtype=torch.int64, device="cuda")
            for rep in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                binding.gemm_f32_valu_probe(form, blocks, iters, out, stamps)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                t = stamps.view(waves, 4).cpu().double()
                mhz = float((100.0 * (t[:, 2] - t[:, 0]) / (t[:, 3] - t[:, 1])).mean())
                fmas = blocks * 256.0 * ((iters // 4) * 64 if form == 2 else iters * 16)
                per_simd_clk = fmas / 64 / (ms * 1e-3) / (cus * 4) / (mhz * 1e6)
                print(json.dumps({"valu_probe_form": form, "operands": what, "waves_per_simd": wps, "run": rep,
                                  "ms": round(ms, 4), "tflops": round(2 * fmas / (ms * 1e-3) / 1e12, 2),
                                  "clock_mhz": round(mhz), "wave64_fma_per_simd_per_clock": round(per_simd_clk, 4),
                                  "tflops_at_2400mhz_same_rate": round(per_simd_clk * 64 * 2 * cus * 4 * 2.4e9 / 1e12, 1)}),
                      flush=True)
    return 0


def lds_probe_cases():
    """(name, form, 64 byte offsets) of the LDS read probe, in launch order.
    Pairs: two groups of lanes on the same banks at different addresses,
    every other lane on one broadcast address in other banks; the pair
    conflicts if and only if one read cycle serves both groups.
      128-bit reads (form 2): every pair of 4-lane quads (lanes 4q .. 4q + 3);
      64-bit reads, plain (form 1) and transposed (form 3): every pair of
      8-lane groups.
    Then the k-contiguous tile reads of the 16 x 16 x 32 kernels (lane l:
    row l % 16, 16-byte chunk l / 16) in three layouts."""
    cases = [("b128 all lanes on one address", 2, [240] * 64),
             ("b128 1 KB contiguous", 2, [16 * l for l in range(64)])]
    for qa in range(16):
        for qb in range(qa + 1, 16):
            offs = [240] * 64
            for i in range(4):
                offs[4 * qa + i] = 1024 + 16 * i
                offs[4 * qb + i] = 2048 + 16 * i
            cases.append((f"b128 quads {qa} {qb}", 2, offs))
    for form, what in ((1, "b64"), (3, "b64_tr_b16")):
        for ga in range(8):
            for gb in range(ga + 1, 8):
                offs = [248] * 64
                for i in range(8):
                    offs[8 * ga + i] = 1024 + 8 * i
                    offs[8 * gb + i] = 2048 + 8 * i
                cases.append((f"{what} groups {ga} {gb}", form, offs))
    rows = lambda pitch, swz: [pitch * (l % 16) + 16 * ((l // 16) ^ swz(l % 16)) for l in range(64)]
    cases.append(("b128 rows of 64 bytes, chunk c ^ ((r / 4) mod 4)", 2, rows(64, lambda r: (r >> 2) & 3)))
    cases.append(("b128 rows of 64 bytes, chunk c ^ 2 ((r / 8) mod 2)", 2, rows(64, lambda r: 2 * ((r >> 3) & 1))))
    cases.append(("b128 rows of 128 bytes, chunk c ^ ((r / 2) mod 8)", 2, rows(128, lambda r: (r >> 1) & 7)))
    return cases


def bench_lds_probe(args) -> int:
    """Launches the LDS read probe once per case (64 reads per lane each),
    printing the cases in launch order; the bank-conflict counts come from a
    profiler run around this command (SQ_LDS_BANK_CONFLICT per dispatch)."""
    import torch

    from shared_memory_tiled_amd import binding

    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    for i, (name, form, offs) in enumerate(lds_probe_cases()):
        t = torch.tensor(offs, dtype=torch.int32, device="cuda")
        binding.gemm_f32_lds_probe(form, t, 64, out)
        torch.cuda.synchronize()
        print(json.dumps({"lds_probe_dispatch": i, "form": form, "case": name}), flush=True)
    return 0


def bench_copy_rate(args) -> int:
    """The rate at which each CU brings 1 KB wave loads from an L2-resident
    buffer, into LDS (the 16-bit kernels' copies) and into registers, from
    the library's measurement helper: one workgroup of 4 waves per CU, each
    with its own 64 KB (2 MB per XCD in all), three runs of each mode; bytes
    per clock per CU from each wave's shader clock cycles."""
    import statistics

    import torch

    from shared_memory_tiled_amd import binding

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    src = torch.randint(0, 1 << 30, (cus * 65536 // 4,), dtype=torch.int32, device="cuda")
    out = torch.zeros(cus * 256, dtype=torch.int32, device="cuda")
    cycles = torch.zeros(cus * 4, dtype=torch.int64, device="cuda")
    nbytes = cus * 4 * iters * 8 * 1024
    for mode, what in ((0, "into LDS"), (1, "into registers")):
        binding.gemm_f32_copy_probe(mode, cus, 2, src, out, cycles)       # warm the caches
        for rep in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            binding.gemm_f32_copy_probe(mode, cus, iters, src, out, cycles)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            cyc = statistics.median(cycles.cpu().tolist())
            print(json.dumps({"copy_probe_mode": mode, "loads": what, "run": rep, "ms": round(ms, 4),
                              "TB_per_s_all_CUs": round(nbytes / ms / 1e9, 2),
                              "bytes_per_clock_per_CU": round(nbytes / cus / cyc, 1),
                              "clock_GHz": round(cyc / (ms * 1e-3) / 1e9, 3)}), flush=True)
    return 0


def bench_ksplit_timeline(args) -> int:
    """Where the k-split kernel's time goes at a workload it runs (default
    square1000), from the library's timeline helper: gemm_f32 runs untimed
    for the settle time, then 20 launches back to back, then -- with no wait
    in between -- the timeline instantiation of the same kernel, whose
    result must have gemm_f32's bits.  Per wave (100 MHz real-time counter):
    start relative to the first wave's start, the wait for its first phase,
    the phase loop, the time to the barrier before the partial tiles are
    added, the sum and the store until the stores have completed, and the
    shader clock over its lifetime.  Medians (and extremes) over all waves."""
    import statistics

    import torch

    from shared_memory_tiled_amd import binding, inputs

    name = args.workload if args.workload != DEFAULT_WORKLOAD else "square1000"
    w = inputs.WORKLOADS[name]
    A, B = inputs.operands(w)
    a = torch.from_numpy(A.buf).cuda()
    b = torch.from_numpy(B.buf).cuda()
    c = torch.empty(w.offset + w.M * w.ldc + 64, dtype=torch.float32, device="cuda")
    call = (w.M, w.N, w.K, a.data_ptr() + 4 * w.offset, w.lda, b.data_ptr() + 4 * w.offset, w.ldb,
            c.data_ptr() + 4 * w.offset, w.ldc)
    handle = torch.cuda.current_stream().cuda_stream
    blocks = ((w.M + 63) // 64) * ((w.N + 63) // 64)
    tl = torch.zeros(32 * blocks, dtype=torch.int32, device="cuda")
    settle(lambda: binding.gemm_f32(*call, handle), args.settle_s)
    for _ in range(20):
        binding.gemm_f32(*call, handle)
    torch.cuda.synchronize()
    ref = c.clone()
    for _ in range(20):
        binding.gemm_f32(*call, handle)
    binding.gemm_f32_ksplit_timeline(*call, tl, tl.numel(), handle)
    torch.cuda.synchronize()
    same_bits = bool(torch.equal(c, ref))
    rows = tl.view(-1, 8).cpu().numpy().astype("int64") & 0xFFFFFFFF
    t0 = rows[:, 0].min()
    us = lambda x: float(x) / 100.0                  # 100 MHz ticks -> microseconds
    parts = {"start_after_first_wave": rows[:, 0] - t0, "first_phase_wait": rows[:, 1] - rows[:, 0],
             "phase_loop": rows[:, 2] - rows[:, 1], "to_partial_barrier": rows[:, 3] - rows[:, 2],
             "sum_and_store": rows[:, 4] - rows[:, 3], "wave_lifetime": rows[:, 4] - rows[:, 0],
             "end_after_first_wave": rows[:, 4] - t0}
    clock = rows[:, 5] / ((rows[:, 4] - rows[:, 0]) / 100e6) / 1e9
    line = {"ksplit_timeline": name, "M": w.M, "N": w.N, "K": w.K, "blocks": blocks, "waves": int(rows.shape[0]),
            "phases_per_wave": sorted(set(int(x) for x in rows[:, 6])), "same_bits_as_gemm_f32": same_bits,
            "clock_GHz_median": round(float(statistics.median(clock)), 3)}
    for k, v in parts.items():
        line[k + "_us"] = {"min": round(us(v.min()), 2), "median": round(us(statistics.median(v)), 2),
                           "max": round(us(v.max()), 2)}
    print(json.dumps(line), flush=True)
    return 0 if same_bits else 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_all_workloads(args) -> int:
    """gemm_f32 (the default kernel) at every workload, then the oracle.

    GPU: 3 warm-up launches, then the timed launches in ten windows, with a
    HIP event on the launch stream before the first window and after each
    (the stream handle is passed to every call; a Python event record after
    every launch would take longer than the microsecond-scale products); the
    median and best per-launch time over the windows give TFLOP/s and the
    fraction of the fp32 peak.  The same number of launches is also captured
    in one HIP graph and replayed (see graph_ms_per_launch), so that they run
    back to back with no host in between.
    Oracle, on this host, unchanged: the full product at square256 and
    square1000 on one thread and on all cores, at square4096 on all cores;
    at the two largest workloads the 4096 sampled entries plus edge entries
    that the parity tests check (one thread), with the full product's time
    extrapolated from that rate and labelled as such."""
    import statistics

    import torch

    from shared_memory_tiled_amd import binding, inputs

    import dataclasses

    cores = len(os.sched_getaffinity(0))
    dev = torch.device("cuda:0")
    runs = []
    for name, launches in WORKLOAD_LAUNCHES.items():
        w = inputs.WORKLOADS[name]
        runs.append((name, launches, w))
        if w.offset != 0:       # the same shape with aligned views: alignment apart from ld
            runs.append((name, launches, dataclasses.replace(w, offset=0)))
    for name, launches, w in runs:
        A, B = inputs.operands(w)
        a = torch.from_numpy(A.buf).to(dev)
        b = torch.from_numpy(B.buf).to(dev)
        c = torch.empty(w.offset + w.M * w.ldc + 64, dtype=torch.float32, device=dev)
        call = (w.M, w.N, w.K, a.data_ptr() + 4 * w.offset, w.lda,
                b.data_ptr() + 4 * w.offset, w.ldb, c.data_ptr() + 4 * w.offset, w.ldc)
        stream = torch.cuda.current_stream()       # the stream the library launches on
        handle = stream.cuda_stream
        settle(lambda: binding.gemm_f32(*call, handle))
        for _ in range(3):
            binding.gemm_f32(*call, handle)
        torch.cuda.synchronize()
        # ten windows of launches between events: a Python event record after
        # every launch takes longer than a microsecond-scale kernel
        per = max(1, launches // 10)
        windows = launches // per
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(windows + 1)]
        ev[0].record(stream)
        for i in range(windows):
            for _ in range(per):
                binding.gemm_f32(*call, handle)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = [ev[i].elapsed_time(ev[i + 1]) / per for i in range(windows)]
        eager_c = c.clone()
        graph = graph_ms_per_launch(lambda: binding.gemm_f32(*call), launches)
        torch.cuda.synchronize()
        graph_same_bits = bool(torch.equal(c, eager_c))
        flop = 2.0 * w.M * w.N * w.K
        med, best = statistics.median(ms), min(ms)
        gmed = statistics.median(graph)
        line = {"workload": name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda, "ldb": w.ldb,
                "ldc": w.ldc, "view_offset_floats": w.offset, "values": w.dist,
                "kernel": binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(w.M, w.N, w.K)),
                "launches": launches, "launches_per_window": per, "median_ms": round(med, 5), "best_ms": round(best, 5),
                "tflops_median": round(flop / med / 1e9, 3), "tflops_best": round(flop / best / 1e9, 3),
                "percent_of_peak_median": round(100 * flop / med / 1e9 / PEAK_FP32_TFLOPS, 2),
                "graph_ms_per_launch": round(gmed, 5), "graph_tflops": round(flop / gmed / 1e9, 3),
                "graph_percent_of_peak": round(100 * flop / gmed / 1e9 / PEAK_FP32_TFLOPS, 2),
                "graph_result_same_bits_as_eager": graph_same_bits}
        del eager_c
        del a, b, c
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline and w.offset == inputs.WORKLOADS[name].offset:
            import oracle
            cpu = {"cores": cores, "cpu": cpu_model()}
            if not w.sampled:
                for threads in (1, cores):
                    t0 = time.perf_counter()
                    oracle.gemm(A.view, B.view, threads=threads)
                    cpu[f"full_s_{threads}_threads"] = round(time.perf_counter() - t0, 3)
            elif name == "square4096":
                t0 = time.perf_counter()
                oracle.gemm(A.view, B.view, threads=cores)
                cpu[f"full_s_{cores}_threads"] = round(time.perf_counter() - t0, 3)
            else:
                ii, jj = inputs.sample_pairs(w.M, w.N, 4096, inputs.rng(w.index, 4))
                t0 = time.perf_counter()
                oracle.gemm_entries(A.view, B.view, ii, jj)
                dt = time.perf_counter() - t0
                cpu["sample_entries"] = int(ii.shape[0])
                cpu["sample_s_1_thread"] = round(dt, 3)
                cpu["full_s_1_thread_extrapolated"] = round(dt * w.M * w.N / ii.shape[0], 1)
            line["oracle"] = cpu
        print(json.dumps(line), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", type=int, default=None, help="time gemm_f32_variant(v) instead")
    ap.add_argument("--ladder", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="NN", choices=["NN", "TN", "NT", "TT"])
    ap.add_argument("--row", default="gemm", choices=["gemm", "transpose", "reduce", "mixed"])
    ap.add_argument("--format", default="bf16", choices=["bf16", "f16"], help="16-bit format of --row mixed")
    ap.add_argument("--n", type=int, default=2 ** 28, help="values summed by --row reduce")
    ap.add_argument("--all-workloads", action="store_true")
    ap.add_argument("--ksplit-timeline", action="store_true",
                    help="per-wave timeline of the k-split kernel at --workload (default square1000)")
    ap.add_argument("--copy-rate", action="store_true",
                    help="per-CU rate of 1 KB wave loads from L2 into LDS and into registers")
    ap.add_argument("--lds-probe", action="store_true",
                    help="launch the LDS read probe over its lane-grouping cases (for a counter run)")
    ap.add_argument("--valu-probe", action="store_true",
                    help="issue rate of non-packed v_fmac_f32 (the register-blocked rung's instruction)")
    ap.add_argument("--shape-sweep", action="store_true")
    ap.add_argument("--shapes", default=None, help="--shape-sweep on these MxNxK shapes (comma separated) only")
    ap.add_argument("--settle-s", type=float, default=None,
                    help="untimed run of each timed step, in seconds, before its warm-up steps "
                         f"(default {SETTLE_S}; {HEADLINE_SETTLE_S} for the headline line)")
    ap.add_argument("--variants", default=None,
                    help="with --ladder: comma-separated variant numbers to time (default: all)")
    ap.add_argument("--view-offset", type=int, default=None,
                    help="floats between each allocation's start and its matrix view "
                         "(default: the workload's own)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="--row transpose: distinct input/output pairs cycled through, so each "
                         "launch reads a matrix the last-level cache no longer holds (1: the same "
                         "matrix every launch)")
    args = ap.parse_args(argv)
    headline = not (args.all_workloads or args.shape_sweep or args.ladder or args.valu_probe or args.lds_probe
                    or args.copy_rate or args.ksplit_timeline or args.row != "gemm")
    if args.settle_s is not None:
        globals()["SETTLE_S"] = max(0.0, args.settle_s)
    elif headline:
        globals()["SETTLE_S"] = HEADLINE_SETTLE_S

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    from shared_memory_tiled_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n}), flush=True)
        del src, dst

    if args.valu_probe:
        return bench_valu_probe(args)
    if args.lds_probe:
        return bench_lds_probe(args)
    if args.ksplit_timeline:
        return bench_ksplit_timeline(args)
    if args.copy_rate:
        return bench_copy_rate(args)
    if args.all_workloads:
        return bench_all_workloads(args)
    if args.shape_sweep:
        return bench_shape_sweep(args)
    if args.row == "reduce":
        return bench_reduce(args)
    w = inputs.WORKLOADS[args.workload]
    if args.view_offset is not None:
        import dataclasses
        w = dataclasses.replace(w, offset=args.view_offset)
    if args.row == "transpose":
        return bench_transpose(args, w)
    if args.row == "mixed":
        return bench_mixed(args, w)
    op_a, op_b = args.op[0], args.op[1]
    if args.op == "NN":
        A, B = inputs.operands(w)
        lda, ldb = w.lda, w.ldb
    else:       # the transposed factor is stored transposed (compact rows)
        ga, gb = inputs.rng(w.index, 0), inputs.rng(w.index, 1)
        A = inputs.padded(inputs.random_matrix(ga, w.K, w.M, w.dist), w.M, w.offset) if op_a == "T" \
            else inputs.padded(inputs.random_matrix(ga, w.M, w.K, w.dist), w.lda, w.offset)
        B = inputs.padded(inputs.random_matrix(gb, w.N, w.K, w.dist), w.K, w.offset) if op_b == "T" \
            else inputs.padded(inputs.random_matrix(gb, w.K, w.N, w.dist), w.ldb, w.offset)
        lda, ldb = A.ld, B.ld
    dev = torch.device("cuda:0")
    a = torch.from_numpy(A.buf).to(dev)
    b = torch.from_numpy(B.buf).to(dev)
    c = torch.empty(w.offset + w.M * w.ldc + 64, dtype=torch.float32, device=dev)
    call_args = (w.M, w.N, w.K, a.data_ptr() + 4 * w.offset, lda,
                 b.data_ptr() + 4 * w.offset, ldb, c.data_ptr() + 4 * w.offset, w.ldc)
    flop = 2.0 * w.M * w.N * w.K

    def one(v):
        if args.op != "NN":
            binding.gemm_f32_op(op_a, op_b, *call_args)
        elif v is None:
            binding.gemm_f32(*call_args)
        else:
            binding.gemm_f32_variant(v, *call_args)

    def timed(v, steps, warmup):
        return _timed(lambda: one(v), steps, warmup)

    if args.ladder:
        variants = list(range(binding.gemm_f32_num_variants())) + \
            [binding.DIAGNOSTIC_BASE + d for d in range(binding.gemm_f32_num_diagnostic_variants())]
        if args.variants:
            variants = [int(v) for v in args.variants.split(",")]
        for v in variants:
            steps = max(1, min(args.steps, 3 if v == 0 else args.steps))
            wall, ms = timed(v, steps, 1)
            print(json.dumps({"variant": v, "name": binding.gemm_f32_variant_name(v),
                              "workload": w.name, "ms_per_launch": round(ms, 4),
                              "tflops": round(flop / ms / 1e9, 2),
                              "frac_of_peak": round(flop / ms / 1e9 / PEAK_FP32_TFLOPS, 4)}), flush=True)
        return 0

    wall, ms_event = timed(args.variant, args.steps, args.warmup)
    value = flop * args.steps / wall / 1e12
    achieved = flop / (ms_event * 1e-3) / 1e12
    kernel_name = binding.gemm_f32_variant_name(binding.gemm_f32_default_variant(w.M, w.N, w.K)
                                                if args.variant is None else args.variant)
    line = {
        "metric": "fp32 GEMM TFLOP/s and % of MI355X fp32 peak at N=4096/8192",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": lda, "ldb": ldb,
                   "ldc": w.ldc, "view_offset_floats": w.offset, "values": w.dist, "op": args.op,
                   "entry_point": (f"gemm_f32_op({op_a},{op_b})" if args.op != "NN" else
                                   "gemm_f32" if args.variant is None else f"gemm_f32_variant({args.variant})"),
                   "kernel": kernel_name, "percent_of_peak": round(100 * value / PEAK_FP32_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name) if args.variant is None and args.op == "NN" else None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(A, B, w, op_a, op_b)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
