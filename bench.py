"""Benchmark: Float8 linear fwd+bwd on one MI355X.

One step = the whole path for every linear of the workload: quantize X, W
and dY (amax, scale, saturating E4M3 cast with the transposed copy), the
forward GEMM and both backward GEMMs, all on device-resident synthetic
inputs (seeded, Llama-3.1-shaped), on one stream (ops.GroupedStep: an X read
by two linears is quantized once, and each linear's GEMMs run as one
grouped launch).  The default workload is the Llama-3.1-8B SwiGLU FFN (w1
and w3: X[8192x4096].W[14336x4096]^T, w2: X[8192x14336].W[4096x14336]^T),
tensorwise scaling.

Prints one JSON line: whole-step TFLOP/s (6*M*N*K per linear), the roofline
of the dominant kernel (the fp8 GEMM, against the dense fp8 MFMA peak)
measured with HIP events on the launch stream around each GEMM launch and
each linear's group of quantizes during the timed steps, the same for the
quantize chain against HBM bandwidth, and the CPU oracle timed on a bounded
sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SOURCES = [os.path.join(ROOT, "float8_mixed_precision_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_schedule.h")]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="ffn8b_tw")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (e.g. under a profiler)")
    p.add_argument("--cpu-rows", type=int, default=640,
                   help="output rows per GEMM in the CPU oracle sample (four times "
                        "as many rows of every quantize input)")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the next_rows measurements (profiling runs of the step alone)")
    p.add_argument("--ffn-block-only", action="store_true",
                   help="only measure the SwiGLU FFN block (profiling runs of its kernels); "
                        "prints its JSON object and exits")
    p.add_argument("--phase-timing", action="store_true",
                   help="only time the GEMM's phases per workgroup (the measurement build "
                        "libfp8phase.so) at the 8B FFN GEMM shapes and exit")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="only run 3 plain device copies of this many bytes (the "
                        "calibration kernel for HBM byte counters) and exit")
    return p.parse_args()


def copy_calibration(nbytes: int):
    """Three launches of a plain streaming elementwise kernel (fp32 negate,
    out of place) over nbytes: nbytes read and nbytes written per launch,
    each touched once, so its HBM byte counters have a known answer."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def gemm_source_hash() -> str:
    """Hash of the GEMM's sources (the kernel and its host-side schedule)."""
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, valid
    only for the workload and the GEMM source the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    if t.get("workload", "").split(" ")[0] != workload:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wl, rows_g: int, rows_q: int = 512):
    """The oracle, as it stands, on a bounded sample of the same step:
    quantize of the first rows_q rows of every input and rows_g output rows
    of every GEMM, each scaled to its full size."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)

    def codes(shape):
        c = rng.integers(0, 256, shape, dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0
        return c

    orc = oracle.default()
    est = 0.0
    flops_sampled = 0
    t_wall = time.perf_counter()
    for lin in wl.linears:
        M, N, K = lin.M, lin.N, lin.K
        for (r, c) in ((M, K), (N, K), (M, N)):
            x = rng.integers(0, 1 << 15, (min(rows_q, r), c), dtype=np.uint16)
            x[(x & 0x7F80) == 0x7F80] = 0
            t = time.perf_counter()
            orc.quantize(x, wl.rowwise)
            est += (time.perf_counter() - t) * r / x.shape[0]
        # (out rows, inner, other operand rows): fwd, grad_x, grad_w
        for (m, k, n) in ((M, K, N), (M, N, K), (N, M, K)):
            a = codes((min(rows_g, m), k))
            b = codes((n, k))
            s = np.ones(1, np.float32)
            t = time.perf_counter()
            orc.gemm_tn(a, s, b, s)
            dt = time.perf_counter() - t
            flops_sampled += 2 * a.shape[0] * n * k
            est += dt * m / a.shape[0]
    wall = time.perf_counter() - t_wall
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": wl.flops / est / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "oracle quantize of %d rows per input and %d output rows per GEMM "
                      "(%.1f GFLOP, %.1f s), each scaled to the full step; estimated "
                      "%.1f s per step" % (rows_q, rows_g, flops_sampled / 1e9, wall, est)}


def measure_e5m2_step(steps, flops_per_step: int, reps: int = 10):
    """The whole step again (same launch plan) with the gradient dY quantized
    to E5M2 and the backward GEMMs reading it so (same buffers, warmed
    first); wall time bracketed by device synchronisation, like `value`."""
    import torch
    from float8_mixed_precision_amd import ops
    for ls in steps:
        ls.e5m2_grad = True
    try:
        grouped = ops.GroupedStep(steps)
        for _ in range(2):
            grouped.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            grouped.run()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
    finally:
        for ls in steps:
            ls.e5m2_grad = False
    v = flops_per_step * reps / el / 1e12
    return {"metric": "whole step, dY in E5M2 (backward GEMMs E5M2 x E4M3)",
            "value": round(v, 2), "unit": "TFLOP/s", "steps": reps,
            "ms_per_step": round(el * 1e3 / reps, 4)}


def measure_pipelined(steps, flops_per_step: int, stream, reps: int = 20):
    """The whole step with each linear's quantizes on a side stream ahead of
    the GEMMs (ops.PipelinedStep): wall time bracketed by device
    synchronisation, then the GEMM groups' event time in further steps (the
    GEMMs share the chip with the next linear's quantizes there)."""
    import torch
    from float8_mixed_precision_amd import ops
    pipe = ops.PipelinedStep(steps, stream)
    for _ in range(3):
        pipe.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        pipe.run()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    rec = []
    for _ in range(5):
        rec += pipe.run(record=True)
    torch.cuda.synchronize()
    g = [(w, n, a.elapsed_time(b)) for k, n, w, a, b in rec if k == "gemm"]
    gt = sum(w for w, _, _ in g) / (sum(t for _, _, t in g) * 1e-3) / 1e12
    return {"metric": "whole step, quantizes of the next linear overlapping the GEMMs",
            "value": round(flops_per_step * reps / el / 1e12, 2), "unit": "TFLOP/s",
            "steps": reps, "ms_per_step": round(el * 1e3 / reps, 4),
            "gemm_achieved_tflops": round(gt, 2), "gemm_frac": round(gt / PEAK_FP8_TFLOPS, 4),
            "gemm_avg_launch_us": round(sum(t for _, _, t in g) * 1e3 / sum(n for _, n, _ in g), 2)}


def measure_ffn_block(steps, wl, stream, reps: int = 5, e5m2_grad: bool = False):
    """The SwiGLU feed-forward block on the FFN workload's tensors (x and W1
    of w1, W3 of w3, W2 and dY of w2): x quantized once for w1 and w3, the
    SwiGLU producers with the amax of h, da, db fused in, nine GEMMs, on one
    stream (the quantizes of the weights and of dY on a side stream measured
    slower: they take power from the GEMMs).  Wall time per step bracketed
    by device synchronisation; HIP events around every launch in further
    steps for the split and the SwiGLU entry points' bandwidth."""
    import torch
    from float8_mixed_precision_amd import ops

    names = [l.name for l in wl.linears]
    if names != ["w1", "w3", "w2"]:
        return None
    w1, w3, w2 = steps[0], steps[1], steps[2]
    blk = ops.SwiGLUFFNStep(w1.x, w1.w, w3.w, w2.w, w2.dy, w1.rowwise, e5m2_grad=e5m2_grad)
    M, D, H = blk.M, blk.D, blk.H
    for _ in range(2):
        blk.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        blk.run()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    # per-launch events, in further steps
    rec = []
    for _ in range(reps):
        rec += [(k, w, None, a, b) for k, w, a, b in blk.run(record=True)]
    torch.cuda.synchronize()
    split = {}
    for kind in ("gemm", "quantize", "swiglu"):
        split[kind] = round(sum(a.elapsed_time(b) for k, _, _, a, b in rec if k == kind) / reps, 4)
    sw = {}
    per = [(w, a.elapsed_time(b)) for k, w, _, a, b in rec if k == "swiglu"]
    for i, name in enumerate(("swiglu_fwd", "swiglu_bwd")):
        v = per[i::2]
        work, ms = v[0][0], sum(t for _, t in v) / len(v)
        ach = work / (ms * 1e-3) / 1e9
        sw[name] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                    "bytes_per_call": work, "avg_call_us": round(ms * 1e3, 2)}
    flops = blk.flops
    # bytes of quantize traffic (amax pass + cast) per step, this block
    # against the same block with x quantized per linear and plain
    # quantizes of h, da, db after a SwiGLU that only writes them
    fused = 6 * M * D * 2 + 18 * H * D + 4 * M * H + 8 * M * H
    unfused = 6 * M * D * 3 + 18 * H * D + 6 * M * H + 12 * M * H
    del blk
    return {"metric": "SwiGLU FFN block fwd+bwd (shared quantize of x, amax fused into the "
                      "SwiGLU producers)%s" % (", gradients E5M2" if e5m2_grad else ""),
            "value": round(flops / wall / 1e12, 2), "unit": "TFLOP/s",
            "shape": {"M": M, "D": D, "H": H}, "flops_per_step": flops, "steps": reps,
            "ms_per_step": round(wall * 1e3, 4), "split_ms_per_step": split, **sw,
            "quantize_bytes_per_step": {"block": fused, "unfused_block": unfused,
                                        "saved_frac": round(1 - fused / unfused, 4)}}


def backlog(cycles: int = 20_000_000):
    """Queue a short device-side spin (about 10 ms) ahead of a group of
    timed launches, so the host enqueues them all before the device reaches
    them: HIP events then time the kernels back to back, not host gaps
    (an idle device records an event as soon as the host enqueues it)."""
    import torch
    torch.cuda._sleep(cycles)


def measure_next_rows(steps, stream, reps: int = 5):
    """The entry points beyond the linear's own step, timed on the same FFN
    tensors after the main measurement (outside `value`): the shard amax and
    the cast with a given scale of Float8 all-gather, and grad_W with an
    fp32 output.  HIP events on the launch stream around every call."""
    import torch
    from float8_mixed_precision_amd import ops

    biggest = max(ls.N * ls.K for ls in steps)
    gw32 = torch.empty(biggest, dtype=torch.float32, device=steps[0].x.device)
    amax_out = torch.empty(1, dtype=torch.float32, device=steps[0].x.device)
    rec = {"amax": [], "quantize_scaled": [], "bwd_w_f32": []}

    def timed(kind, work, fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        rec[kind].append((work, e0, e1))

    for r in range(reps + 1):
        backlog()
        for ls in steps:
            for t, qz in ((ls.x, ls.qx), (ls.w, ls.qw), (ls.dy, ls.qdy)):
                n = t.numel()
                timed("amax", 2 * n, lambda: ops.fp8_linear_amax(t, amax_out, ls.ws))
                timed("quantize_scaled", 4 * n,
                      lambda: ops.fp8_linear_quantize_scaled(t, qz.scale, qz.q, qz.qt))
            g = gw32[:ls.N * ls.K].view(ls.N, ls.K)
            timed("bwd_w_f32", 2 * ls.M * ls.N * ls.K,
                  lambda: ops.fp8_linear_bwd_w_f32(ls.qdy.qt, ls.qdy.scale_t, ls.qx.qt,
                                                   ls.qx.scale_t, ls.M, ls.N, ls.K,
                                                   ls.rowwise, g))
        if r == 0:                      # first round is warm-up
            torch.cuda.synchronize()
            for v in rec.values():
                v.clear()
    # the cast alone with the Infinity Cache defeated: the step's distinct
    # input tensors (1.19 GB of bf16 at the 8B FFN shape) cast in turn, each
    # with its own scale, so that every cast reads a tensor last touched
    # more than 1 GB of traffic earlier (from HBM, not the 256 MB cache)
    rec["cast_hbm"] = []
    tensors, seen = [], set()
    for ls in steps:
        for t, qz in ((ls.x, ls.qx), (ls.w, ls.qw), (ls.dy, ls.qdy)):
            if t.data_ptr() not in seen:
                seen.add(t.data_ptr())
                tensors.append((t, qz))
    for r in range(reps + 1):
        backlog()
        for t, qz in tensors:
            timed("cast_hbm", 4 * t.numel(),
                  lambda: ops.fp8_linear_quantize_scaled(t, qz.scale, qz.q, qz.qt))
        if r == 0:
            torch.cuda.synchronize()
            rec["cast_hbm"].clear()
    # the shard amax alone in the same rotation (two launches per call:
    # partial maxima, then one workgroup reduces them into amax_out)
    rec["amax_hbm"] = []
    for r in range(reps + 1):
        backlog()
        for t, qz in tensors:
            timed("amax_hbm", 2 * t.numel(),
                  lambda: ops.fp8_linear_amax(t, amax_out, steps[0].ws))
        if r == 0:
            torch.cuda.synchronize()
            rec["amax_hbm"].clear()
    torch.cuda.synchronize()
    out = {"stream_ceiling": measure_stream_ceiling(stream)}
    for kind, v in rec.items():
        work = sum(w for w, _, _ in v)
        ms = sum(a.elapsed_time(b) for _, a, b in v)
        if kind == "bwd_w_f32":
            ach = work / (ms * 1e-3) / 1e12
            out[kind] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                         "calls": len(v), "avg_call_us": round(ms * 1e3 / len(v), 2)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            out[kind] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "bytes_per_element": {"amax": 2, "amax_hbm": 2}.get(kind, 4),
                         "calls": len(v), "avg_call_us": round(ms * 1e3 / len(v), 2)}
    ceil = out["stream_ceiling"]
    out["amax_hbm"]["frac_of_read_ceiling"] = round(out["amax_hbm"]["achieved"]
                                                    / ceil["read"]["achieved"], 4)
    out["cast_hbm"]["frac_of_copy_ceiling"] = round(out["cast_hbm"]["achieved"]
                                                    / ceil["copy"]["achieved"], 4)
    out["amax"]["note"] = ("interleaved with the given-scale casts and fp32 grad_W GEMMs of "
                           "the same tensors: each amax pays for the previous cast's dirty "
                           "lines; amax_hbm is the shard amax alone")
    return out


def measure_stream_ceiling(stream, nbytes: int = 1 << 30, workgroups: int = 2048,
                           reps: int = 5):
    """Hand-written 16-byte streaming kernels (libfp8probe's fp8_probe_stream)
    over 1 GiB buffers, four times the Infinity Cache: read only, write only,
    and copy.  Median of reps launches each (HIP events on the launch
    stream); they are the practical ceilings of the amax pass (read) and the
    cast (as many bytes read as written)."""
    import ctypes
    import torch
    from float8_mixed_precision_amd import build as B

    L = ctypes.CDLL(B.PROBE_PATH)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8_probe_stream.restype = I
    L.fp8_probe_stream.argtypes = [I, P, P, i64, I, P, P]
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda:0")
    hs = ctypes.c_void_p(stream.cuda_stream)
    out = {"kernel": "fp8_probe_stream: grid-stride, 16-byte accesses, 8 in flight per "
                     "thread, %d workgroups of 256 threads" % workgroups,
           "bytes": nbytes, "unit": "GB/s", "peak": PEAK_HBM_GBS}
    for name, kind, factor in (("read", 0, 1), ("write", 1, 1), ("copy", 2, 2)):
        ts = []
        for r in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            backlog()
            e0.record(stream)
            if L.fp8_probe_stream(kind, src.data_ptr(), dst.data_ptr(), nbytes, workgroups,
                                  sink.data_ptr(), hs) != 0:
                raise RuntimeError("fp8_probe_stream failed")
            e1.record(stream)
            torch.cuda.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        v = factor * nbytes / (ms * 1e-3) / 1e9
        out[name] = {"achieved": round(v, 1), "frac": round(v / PEAK_HBM_GBS, 4)}
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def measure_workload_step(name: str, reps: int = 20, warmup_s: float = 0.3,
                          min_timed_s: float = 0.1):
    """The whole step of another workload (its own seeded tensors, freed
    afterwards), timed like `value`, with the GEMM and quantize-chain
    rooflines from the same kind of HIP events.  The warm-up runs for
    warmup_s seconds (the tensors are generated on the host first, and the
    GPU comes out of that idle at a low clock), and at least min_timed_s
    seconds of steps are timed."""
    import torch
    from float8_mixed_precision_amd import ops
    from float8_mixed_precision_amd import workloads as W

    wl = W.WORKLOADS[name]
    dev = torch.device("cuda:0")
    data = W.generate(wl)
    steps, shared, qx_of = [], {}, {}
    for lin, d in zip(wl.linears, data):
        key = id(d["x"])
        if key not in shared:
            shared[key] = W.bits_to_torch(d["x"], dev)
        steps.append(ops.LinearStep(shared[key], W.bits_to_torch(d["w"], dev),
                                    W.bits_to_torch(d["dy"], dev), wl.rowwise,
                                    qx=qx_of.get(key)))
        qx_of.setdefault(key, steps[-1].qx)
    del data
    grouped = ops.GroupedStep(steps)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < warmup_s:
        for _ in range(4):
            grouped.run()
        torch.cuda.synchronize()
        n += 4
    per_step = (time.perf_counter() - t0) / n
    reps = max(reps, int(min_timed_s / per_step) + 1)
    evs = []
    t0 = time.perf_counter()
    for _ in range(reps):
        evs += grouped.run(record=True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    g_fl = sum(w for k, _, w, _, _ in evs if k == "gemm")
    g_ms = sum(a.elapsed_time(b) for k, _, _, a, b in evs if k == "gemm")
    q_b = sum(w for k, _, w, _, _ in evs if k == "quantize")
    q_ms = sum(a.elapsed_time(b) for k, _, _, a, b in evs if k == "quantize")
    gt = g_fl / (g_ms * 1e-3) / 1e12
    qg = q_b / (q_ms * 1e-3) / 1e9
    out = {"workload": wl.name, "description": wl.description,
           "scaling": "rowwise" if wl.rowwise else "tensorwise",
           "value": round(wl.flops * reps / el / 1e12, 2), "unit": "TFLOP/s",
           "steps": reps, "ms_per_step": round(el * 1e3 / reps, 4),
           "gemm": {"bound": "mfma", "achieved": round(gt, 2), "peak": PEAK_FP8_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(gt / PEAK_FP8_TFLOPS, 4)},
           "quantize": {"bound": "hbm", "achieved": round(qg, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(qg / PEAK_HBM_GBS, 4),
                        "bytes_per_element": 6},
           "time_split_ms_per_step": {"gemm": round(g_ms / reps, 4),
                                      "quantize": round(q_ms / reps, 4)}}
    del steps, shared, grouped, evs
    torch.cuda.empty_cache()
    return out


def measure_per_layout(steps, stream, reps: int = 5):
    """Each GEMM of the step launched alone (one fp8_linear_gemm_grouped
    problem per launch, same kernel as the step), HIP events around every
    launch: TFLOP/s per layout (fwd X.W^T, grad_X dY.W, grad_W dY^T.X), per
    linear and summed over the linears.  Run after the timed steps; the
    step itself launches them grouped."""
    import torch
    from float8_mixed_precision_amd import ops
    kinds = {
        "fwd": lambda ls: (ls.qx.q, ls.qx.scale, ls.qw.q, ls.qw.scale, ls.out, ls.K),
        "grad_x": lambda ls: (ls.qdy.q, ls.qdy.scale, ls.qw.qt, ls.qw.scale_t, ls.grad_x, ls.N),
        "grad_w": lambda ls: (ls.qdy.qt, ls.qdy.scale_t, ls.qx.qt, ls.qx.scale_t, ls.grad_w,
                              ls.M),
    }
    rec = []
    for r in range(reps + 1):
        backlog()
        for li, ls in enumerate(steps):
            for kind, f in kinds.items():
                a, sa, b, sb, c, k = f(ls)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                ops.fp8_linear_gemm_grouped([(a, sa, b, sb, c)], ls.rowwise, stream,
                                            e5m2=ls.e5m2_grad and kind != "fwd")
                e1.record(stream)
                if r:
                    rec.append((li, kind, 2 * ls.M * ls.N * ls.K, k, e0, e1))
        if r == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    out = {"method": "each GEMM alone, HIP events per launch, %d launches per GEMM" % reps}
    for kind in kinds:
        sel = [x for x in rec if x[1] == kind]
        fl = sum(x[2] for x in sel)
        ms = sum(x[4].elapsed_time(x[5]) for x in sel)
        per = []
        for li in range(len(steps)):
            s2 = [x for x in sel if x[0] == li]
            ms2 = sum(x[4].elapsed_time(x[5]) for x in s2)
            per.append({"linear": li, "contraction": s2[0][3],
                        "tflops": round(sum(x[2] for x in s2) / (ms2 * 1e-3) / 1e12, 1)})
        out[kind] = {"tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                     "per_linear": per}
    return out


def collect_step_samples(steps, per_gemm: int = 1536, seed: int = 7):
    """Host copies of what the CPU oracle needs to check the timed step's
    results: every fp8 operand and scale as the device wrote it, the bf16
    inputs, and sampled outputs of each GEMM (random positions plus the
    corners of the output).  Plain data movement, no arithmetic."""
    import numpy as np
    import torch
    rng = np.random.default_rng(seed)

    def h(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    torch.cuda.synchronize()
    lins = []
    for ls in steps:
        d = {"rowwise": ls.rowwise, "M": ls.M, "N": ls.N, "K": ls.K}
        for name, qz, src in (("x", ls.qx, ls.x), ("w", ls.qw, ls.w), ("dy", ls.qdy, ls.dy)):
            d[name] = (h(qz.q), h(qz.qt), h(qz.scale), h(qz.scale_t), h(src))
        for kind, t in (("fwd", ls.out), ("grad_x", ls.grad_x), ("grad_w", ls.grad_w)):
            m, n = t.shape
            ii = np.concatenate([rng.integers(0, m, per_gemm), [0, 0, m - 1, m - 1]])
            jj = np.concatenate([rng.integers(0, n, per_gemm), [0, n - 1, 0, n - 1]])
            d[kind] = (ii, jj, h(t)[ii, jj])
        lins.append(d)
    return lins


def step_parity(lins, rows_per_tensor: int = 8, seed: int = 11):
    """The oracle on the timed step's data (CPU leg): the sampled GEMM outputs
    against the oracle's GEMM on the device's own fp8 operands (relative
    Frobenius, largest bf16 ulp distance, share within 2 ulps), and the
    quantize of sampled rows against the oracle's (the scale from the amax
    of the whole bf16 tensor, then the cast of those rows with it: the bytes
    must be equal).  Tensorwise workloads check q and qt rows; rowwise
    workloads check the scale vectors only."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    G, O = [], []
    q_rows = q_bad = 0
    for d in lins:
        for name in ("x", "w", "dy"):
            q, qt, sc, sct, x = d[name]
            a = oracle.amax(x)
            if d["rowwise"]:
                continue
            s_or = oracle.scale_from_amax(a)
            if np.float32(s_or).view(np.uint32) != sc.view(np.uint32)[0]:
                q_bad += 1
            rows = rng.integers(0, x.shape[0], rows_per_tensor)
            for r in rows:
                rq, _ = oracle.quantize_scaled(x[r:r + 1], sc[0])
                q_rows += 1
                q_bad += int(not np.array_equal(rq.ravel(), q[r]))
            # columns of x = rows of qt
            cols = rng.integers(0, x.shape[1], rows_per_tensor)
            for c in cols:
                q_rows += 1
                q_bad += int(not np.array_equal(q[:, c], qt[c]))
        operands = {"fwd": (d["x"][0], d["x"][2], d["w"][0], d["w"][2]),
               "grad_x": (d["dy"][0], d["dy"][2], d["w"][1], d["w"][3]),
               "grad_w": (d["dy"][1], d["dy"][3], d["x"][1], d["x"][3])}
        for kind, (a, sa, b, sb) in operands.items():
            ii, jj, g = d[kind]
            O.append(oracle.gemm_tn_sampled(a, sa, b, sb, ii, jj))
            G.append(g)
    G = np.concatenate(G)
    O = np.concatenate(O)
    dist = oracle.bf16_ulp_distance(G, O)
    return {"gemm_outputs_sampled": int(len(G)),
            "relfro": float("%.3g" % oracle.rel_frobenius(G, O)),
            "max_ulp": int(dist.max()), "frac_le2": round(float(np.mean(dist <= 2)), 6),
            "quantize_rows_checked": q_rows, "quantize_rows_differing": q_bad,
            "note": "GEMM outputs of the last timed step against the oracle's GEMM on the "
                    "device's fp8 operands; quantize rows (and q/qt transposes) against the "
                    "oracle's cast with the scale of the tensor's amax"}


def environment():
    """ROCm / HIP version, the device's architecture and compute units."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"hip": torch.version.hip, "torch": torch.__version__,
            "gfx_arch": getattr(p, "gcnArchName", None), "device": p.name,
            "compute_units": p.multi_processor_count}


def measure_mfma_ceiling(codes, stream, target_ms: float = 25.0, launches: int = 4):
    """The fp8 MFMA instruction alone (libfp8probe's k_mfma_loop: register
    operands, the GEMM's 8 x 8 accumulator layout and snake order, no
    memory traffic) on one workgroup per compute unit, timed with HIP events
    over `launches` launches of about target_ms each: on the step's own
    E4M3 codes, and on all-zero codes (the least switching).  The first is
    the rate the GEMM's main loop could reach on this data under the board's
    power limit."""
    import ctypes
    import torch
    from float8_mixed_precision_amd import build as B

    L = ctypes.CDLL(B.PROBE_PATH)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8_probe_mfma_loop.restype = I
    L.fp8_probe_mfma_loop.argtypes = [P, i64, I, I, P, P]
    wg, per_wg = 256, 4 * 512 * 2 * 16 * 16 * 128      # flops per workgroup per iteration
    sink = torch.empty(wg * 256, dtype=torch.float32, device=codes.device)
    zeros = torch.zeros(1 << 20, dtype=torch.uint8, device=codes.device)
    hs = ctypes.c_void_p(stream.cuda_stream)

    def run(buf, iters, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            if L.fp8_probe_mfma_loop(buf.data_ptr(), buf.numel(), wg, iters,
                                     sink.data_ptr(), hs) != 0:
                raise RuntimeError("fp8_probe_mfma_loop failed")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    ms = run(codes, 200, 1)
    iters = max(200, int(200 * target_ms / max(ms, 1e-3)))
    out = {"kernel": "k_mfma_loop: v_mfma_f32_16x16x128_f8f6f4 on register operands, "
                     "one 256-thread workgroup per compute unit", "unit": "TFLOP/s",
           "peak": PEAK_FP8_TFLOPS, "iters": iters, "launches": launches}
    for name, buf in (("e4m3_codes", codes), ("zero_codes", zeros)):
        run(buf, iters, 1)
        t = run(buf, iters, launches)
        v = wg * per_wg * iters * launches / (t * 1e-3) / 1e12
        out[name] = {"achieved": round(v, 1), "frac": round(v / PEAK_FP8_TFLOPS, 4)}
    return out


def measure_board(run_step, seconds: float = 2.5):
    """Engine clock and board power while the step runs back to back for
    `seconds` (the driver's averaged readings through torch.cuda /
    amdsmi, sampled every 50 ms over the second half of the run, when the
    readings reflect the load; they lag the load by a few hundred ms).
    Returns None where the readings are unavailable."""
    import threading
    import torch
    try:
        torch.cuda.clock_rate(0)
        torch.cuda.power_draw(0)
    except Exception:
        return None
    samples, phase, stop = [], ["idle"], [False]

    def sampler():
        while not stop[0]:
            try:
                samples.append((phase[0], time.perf_counter(), float(torch.cuda.clock_rate(0)),
                                float(torch.cuda.power_draw(0))))
            except Exception:
                pass
            time.sleep(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    phase[0] = "load"
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            run_step()
            n += 1
        torch.cuda.synchronize()
    t1 = time.perf_counter()
    stop[0] = True
    th.join()
    load = [s for s in samples if s[0] == "load" and s[1] >= t0 + (t1 - t0) / 2]
    if not load:
        return None
    mean = lambda xs: round(sum(xs) / len(xs), 1)
    return {"clock_mhz": mean([s[2] for s in load]),
            "power_w": mean([s[3] for s in load]),
            "power_w_max": max(s[3] for s in load),
            "samples": len(load), "steps": n, "seconds": round(t1 - t0, 2),
            "source": "torch.cuda.clock_rate / power_draw (amdsmi averages) while the step "
                      "runs back to back"}


def phase_timing():
    """Per-tile phases of the persistent GEMM (libfp8phase.so: the same
    kernels with shader-clock and 100 MHz real-time counters read at a
    tile's top, after its first k-tile, after its last k-tile and after its
    last store is issued) for the forward, grad_X and grad_W shapes of the
    8B FFN's w1, each launched back to back on E4M3 codes of N(0,1)
    activations and N(0,0.02) weights quantized by this library.  Medians
    over the tiles of the last launch; the gap is from a tile's last store to
    the top of the same workgroup's next tile, the period from one tile's top
    to the next's; the clock is shader cycles over real time."""
    import ctypes
    import numpy as np
    import torch
    from float8_mixed_precision_amd import build as B
    from float8_mixed_precision_amd import ops

    ops.LIB_PATH = B.PHASE_PATH
    L = ops.lib()
    L.fp8_gemm_phase_read.restype = ctypes.c_int
    L.fp8_gemm_phase_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    out = []
    for name, (M, N, K) in (("fwd", (8192, 14336, 4096)), ("grad_x", (8192, 4096, 14336)),
                            ("grad_w", (14336, 4096, 8192))):
        a = (torch.randn(M, K, device=dev, generator=gen)).to(torch.bfloat16)
        b = (torch.randn(N, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        qa, qb = ops.fp8_linear_quantize(a), ops.fp8_linear_quantize(b)
        o = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        launch = lambda: ops.fp8_linear_gemm_grouped([(qa.q, qa.scale, qb.q, qb.scale, o)])
        for _ in range(30):
            launch()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            launch()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        nb = (M // 256) * (N // 256)
        buf = np.zeros(nb * 8, dtype=np.uint64)
        if L.fp8_gemm_phase_read(buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("fp8_gemm_phase_read failed")
        d = buf.reshape(nb, 8).astype(np.int64)
        t0, r0, ta, ra, t1, r1, t2, r2 = (d[:, i] for i in range(8))
        nk = K // 128
        G = min(nb, 256)                  # workgroups; record s + G is the next tile of s's
        clk = (t2 - t0) / ((r2 - r0) / 100e6) / 1e9
        loop = float(np.median(t1 - ta))
        period = float(np.median(t0[G:] - t0[:-G]))
        out.append({"gemm": name, "M_N_K": [M, N, K], "tiles": nb, "workgroups": G,
                    "avg_launch_us": round(us, 1),
                    "tflops": round(2 * M * N * K / us / 1e6, 1),
                    "clock_ghz_median": round(float(np.median(clk)), 3),
                    "clock_ghz_min_max": [round(float(clk.min()), 3), round(float(clk.max()), 3)],
                    "head_cycles": int(np.median(ta - t0)),
                    "loop_cycles_per_ktile": round(loop / (nk - 1), 1),
                    "loop_issue_efficiency": round(2048 * (nk - 1) / loop, 4),
                    "epilogue_cycles": int(np.median(t2 - t1)),
                    "gap_cycles": int(np.median(t0[G:] - t2[:-G])),
                    "tile_period_cycles": int(period),
                    "mfma_share_of_period": round(2048 * nk / period, 4)})
        del a, b, qa, qb, o
    print(json.dumps({"phase_timing": out}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.phase_timing:
        phase_timing()
        return

    import numpy as np
    import torch

    from float8_mixed_precision_amd import ops
    from float8_mixed_precision_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating %s" % wl.name, file=sys.stderr, flush=True)
    data = W.generate(wl)
    steps = []
    shared = {}
    qx_of = {}
    for lin, d in zip(wl.linears, data):
        key = id(d["x"])
        if key not in shared:
            shared[key] = W.bits_to_torch(d["x"], dev)
        # a linear reading the X of an earlier one reuses its quantize
        steps.append(ops.LinearStep(shared[key], W.bits_to_torch(d["w"], dev),
                                    W.bits_to_torch(d["dy"], dev), wl.rowwise,
                                    qx=qx_of.get(key)))
        qx_of.setdefault(key, steps[-1].qx)
    del data
    stream = torch.cuda.current_stream()
    if args.ffn_block_only:
        print("[bench] ffn block only", file=sys.stderr, flush=True)
        print(json.dumps(measure_ffn_block(steps, wl, stream, reps=args.steps)), flush=True)
        return

    # one step on the current stream: per linear its quantizes, forward GEMM
    # and grad_X; the grad_W of w1 and w3 in one grouped launch; timing
    # events around each group of launches, (kind, launches, work, start, end)
    grouped = ops.GroupedStep(steps)

    def run_step(record):
        return grouped.run(stream, record)

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run_step(False)
    torch.cuda.synchronize()

    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    all_evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_evs += run_step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def agg(kind):
        work = sum(w for k, _, w, _, _ in all_evs if k == kind)
        ms = sum(a.elapsed_time(b) for k, _, _, a, b in all_evs if k == kind)
        n = sum(c for k, c, _, _, _ in all_evs if k == kind)
        return work, ms, n

    g_flops, g_ms, g_n = agg("gemm")
    q_bytes, q_ms, q_n = agg("quantize")
    gemm_tflops = g_flops / (g_ms * 1e-3) / 1e12
    quant_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    value = wl.flops * args.steps / elapsed / 1e12

    # host copies of the last timed step's operands and sampled outputs, for
    # the oracle's check in the CPU leg
    samples = None if args.no_cpu_baseline else collect_step_samples(steps)
    traffic = measured_traffic(wl.name)
    result = {
        "metric": "fp8 linear fwd+bwd TFLOP/s at Llama-3.1-8B FFN shape; % fp8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
        "data": "synthetic (seeded numpy draws rounded to bf16; device-resident)",
        "config": {"workload": wl.name, "description": wl.description,
                   "scaling": "rowwise" if wl.rowwise else "tensorwise",
                   "linears": [{"name": l.name, "M": l.M, "N": l.N, "K": l.K}
                               for l in wl.linears],
                   "flops_per_step": wl.flops},
        "pct_fp8_peak_step": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "roofline": {
            "kernel": "k_gemm_fp8_pers (each linear's fwd, grad_x and grad_w in one grouped "
                      "launch; w1's grad_w in w3's)",
            "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "launches": g_n, "avg_launch_us": round(g_ms * 1e3 / g_n, 2),
            "avg_flops_per_launch": g_flops // g_n,
        },
        "roofline_quantize": {
            "kernel": "amax + finalize + cast_transpose chain per tensor",
            "bound": "hbm", "achieved": round(quant_gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(quant_gbs / PEAK_HBM_GBS, 4),
            "bytes_per_element": 6, "calls": q_n, "avg_call_us": round(q_ms * 1e3 / q_n, 2),
            "note": "X of w1 and w3 quantized once",
        },
        "time_split_ms_per_step": {"gemm": round(g_ms / args.steps, 4),
                                   "quantize": round(q_ms / args.steps, 4)},
        "cpu_baseline": None,
        "parity": None,
        "environment": environment(),
    }
    print("[bench] per-layout GEMM rates", file=sys.stderr, flush=True)
    result["gemm_per_layout"] = measure_per_layout(steps, stream)
    if not args.no_next_rows:
        print("[bench] MFMA-only ceiling", file=sys.stderr, flush=True)
        ceil = measure_mfma_ceiling(steps[0].qx.q, stream)
        ceil["gemm_fraction_of_e4m3_ceiling"] = round(gemm_tflops / ceil["e4m3_codes"]["achieved"], 4)
        ceil["codes"] = "the step's E4M3 codes of X (N(0,1) activations scaled onto 448)"
        result["mfma_ceiling"] = ceil
        print("[bench] next rows", file=sys.stderr, flush=True)
        result["next_rows"] = measure_next_rows(steps, stream)
        result["next_rows"]["e5m2_grad_step"] = measure_e5m2_step(steps, wl.flops)
        print("[bench] pipelined step", file=sys.stderr, flush=True)
        result["next_rows"]["pipelined_step"] = measure_pipelined(steps, wl.flops, stream)
        print("[bench] ffn block", file=sys.stderr, flush=True)
        blk = measure_ffn_block(steps, wl, stream)
        if blk is not None:
            result["next_rows"]["ffn_block"] = blk
            result["next_rows"]["ffn_block_e5m2"] = measure_ffn_block(steps, wl, stream,
                                                                      e5m2_grad=True)
    if not args.no_next_rows and args.workload == "ffn8b_tw":
        # its own tensors next to the FFN's (a few GB of 288)
        print("[bench] rowwise outlier step", file=sys.stderr, flush=True)
        result["next_rows"]["rowwise_step"] = measure_workload_step("outlier_rw")
        print("[bench] 8B attention projection and 70B-shaped FFN steps", file=sys.stderr,
              flush=True)
        result["next_rows"]["attn8b_step"] = measure_workload_step("attn8b_tw")
        result["next_rows"]["ffn70b_step"] = measure_workload_step("ffn70b_tw", reps=10)
    if not args.no_next_rows:
        # last of the GPU measurements: 2.5 s of back-to-back steps heat the
        # chip, which would bias whatever is timed after it
        print("[bench] board clock and power", file=sys.stderr, flush=True)
        result["board"] = measure_board(lambda: run_step(False))
    del steps, shared, grouped
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle: parity of the timed step", file=sys.stderr, flush=True)
        result["parity"] = step_parity(samples)
        del samples
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows, 4 * args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
