#!/usr/bin/env python3
"""Benchmark of the accelerator linear layer on one MI355X.

Default line (no --workload): the bf16 prefill, 2048 tokens of x through
two bf16 weights [4096 | 14336] x 4096 in one il_matmul submission -- the
largest configuration that fits one GPU.  One step = one such call.  The K
timed steps are eager calls bracketed by synchronisations (host validation
and launches included); weight copies are rotated so that one rotation
exceeds 1 GiB and every step reads its weights from HBM, not from the
256 MiB last-level cache.  value = TFLOP/s of whole calls.  `roofline` takes
the GEMM kernel alone (median over calls of the HIP events the library
records on the launch stream around each of the call's two kernels, a
512 MiB scratch write before each call) against 2.5 PFLOP/s dense bf16; the
same line carries the call's device time, the graph-replay time per call,
the eager per-call cost beside the pages' ~0.15 ms dispatch figure, the
inputs' SHA-256, the host CPU (the shader clock is not read live: the note
says where the counter bound on it stands, beside one amd-smi clock and
power reading taken under the calls), the il_wants threshold
calibrated from the cost of a launch-bound call and the oracle's rate, a
`cpu_baseline` (the oracle on the host cores, on the first 16 rows of x)
and a `decode` object: weight GB/s against 8 TB/s of the decode workloads
(fused bf16 t = 1, Q8 gate/up and down t = 1, Q4 t = 1, 2, 4, 8), each timed
in a HIP graph of calls, with its eager per-call cost and the oracle's
time over the same submission (median of 3, on one host core and on all).

--workload NAME times one workload alone (graph replay, or eager with
--no-graph) and prints its own line in the same form.  --decode-sweep times
both decode kernel families and the library's choice between them over
model-like shapes; --calibrate-read / --calibrate-copy time a plain read and
a plain copy (the read ceiling and the counter scaling).
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from quantized_weight_matmul_amd import workloads as wl  # noqa: E402

METRIC = "weight GB/s (decode GEMV, % HBM peak); TFLOP/s (prefill GEMM, % MFMA peak)"

def path_dtype(fmts, t):
    """Arithmetic of the kernel family il_matmul runs for these weight formats
    at t tokens (the dispatch in csrc/il_gemv.hip and il_gemm.hip): f32 FMAs on
    the streaming decode kernel (bf16 weights, and Q8 below t = 4); bf16
    matrix-core products with f32 accumulation otherwise (the decode kernel's
    x as two bf16 parts, hi + lo; bf16(x) on the mid-size and GEMM paths)."""
    if t <= 8 and all(f == "bf16" or (f == "q8" and t < 4) for f in fmts):
        return "f32"
    return "bf16"

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk, dense
ROTATE_BYTES = 1 << 30
# Up to this t the call streams the weights once with few flops per byte
# (decode, and the mid-size verify path): weight GB/s against HBM.  Beyond,
# TFLOP/s against the bf16 matrix cores.
STREAMING_MAX_T = 32

DESCRIPTIONS = {
    "c1": "single bf16 job, t=1, [1024, 256]",
    "c2": "fused bf16 decode, t=1, 3 jobs [4096|1024|1024] x 4096",
    "c3a": "Q8 decode, t=1, 2 jobs [14336, 4096] (gate/up)",
    "c3b": "Q8 decode, t=1, 1 job [4096, 14336] (down)",
    "c4_t1": "Q4 verify, t=1, 2 jobs [17408, 5120]",
    "c4_t2": "Q4 verify, t=2, 2 jobs [17408, 5120]",
    "c4_t4": "Q4 verify, t=4, 2 jobs [17408, 5120]",
    "c4_t8": "Q4 verify, t=8, 2 jobs [17408, 5120]",
    "c4_t16": "Q4 verify, t=16, 2 jobs [17408, 5120]",
    "c4_t32": "Q4 verify, t=32, 2 jobs [17408, 5120]",
    "c4_t64": "Q4 verify, t=64, 2 jobs [17408, 5120] (mid-size plan: 64-token units on 4 waves)",
    "c4_t128": "Q4 verify, t=128, 2 jobs [17408, 5120] (mid-size plan: 128-token units)",
    "c5a": "bf16 prefill, t=2048, 2 jobs [4096|14336] x 4096",
    "c5b": "Q4 prefill, t=512, 1 job [14336, 4096]",
    "f4_lmhead_t1": "centroid-masked LM head, t=1: h=256, 2048 centroids, top 32, vocabulary 2^18 (bf16)",
    "f3_q8_t1": "fused gate/up + GELU, Q8, t=1, 2 x [14336, 4096] -> y = GELU(x G^T) * (x U^T)",
    "f3_q4_t1": "fused gate/up + GELU, Q4, t=1, 2 x [14336, 4096] -> y = GELU(x G^T) * (x U^T)",
    "f3_bf16_t1": "fused gate/up + GELU, bf16, t=1, 2 x [14336, 4096] -> y = GELU(x G^T) * (x U^T)",
    "f3_q8_t512": "fused gate/up + GELU, Q8, t=512, 2 x [14336, 4096] -> y = GELU(x G^T) * (x U^T) (prefill GEMM)",
    "f3_q4_t512": "fused gate/up + GELU, Q4, t=512, 2 x [14336, 4096] -> y = GELU(x G^T) * (x U^T) (prefill GEMM)",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(name: str) -> str:
    import hashlib
    path = os.path.join(ROOT, "quantized_weight_matmul_amd", "csrc", name)
    try:
        with open(path, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return ""


def measured_traffic(workload: str, kernel: str | None = None):
    """HBM bytes per launch of the workload's kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (profiles/traffic.json), scaled by
    the same counters on a plain copy of known size; with `kernel`, that
    kernel's own bytes (a call of several kernels); None when absent or when
    a source of the call's kernels changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or not rec.get("kernel_sources"):
        return None
    if any(kernel_source_sha(name) != sha for name, sha in rec["kernel_sources"].items()):
        return None
    if kernel is not None:
        b = rec.get("hbm_bytes_per_kernel", {}).get(kernel)
        return int(b) if b is not None else None
    return int(rec["hbm_bytes_per_launch"])


def cpu_baseline(sub: wl.Submission, x, weights, budget_s: float) -> dict:
    """The oracle, as it stands, on the host cores: a bounded sample of the
    same workload (whole submissions for decode; a slice of x's rows for
    prefill), scaled to the metric's unit, on every core and on one."""
    import oracle
    threads = oracle_threads()
    streaming = sub.t <= STREAMING_MAX_T
    xs = x if streaming else x[:16]

    def timed(n_threads, budget):
        reps = 0
        t0 = time.perf_counter()
        while True:
            for j, w in zip(sub.jobs, weights):
                oracle.matmul(xs, w, j.fmt, j.n_out, threads=n_threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or (el > 0 and el / reps * (reps + 1) > budget * 2):
                return reps, el

    def rate(reps, el):
        per = el / reps
        if streaming:
            return sub.weight_bytes / per / 1e9
        return sum(2 * xs.shape[0] * j.n_out * sub.n_in for j in sub.jobs) / per / 1e12

    reps, el = timed(threads, budget_s)
    reps1, el1 = timed(1, max(1.0, budget_s / 4))
    if streaming:
        unit = "GB/s"
        what = f"full oracle passes over the submission ({sub.weight_bytes / 1e6:.1f} MB of weights each)"
    else:
        unit = "TFLOP/s"
        what = f"oracle passes over the first {xs.shape[0]} rows of x (all jobs)"
    return {"value": round(rate(reps, el), 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{reps} {what}", "seconds": round(el, 2),
            "single_core": {"value": round(rate(reps1, el1), 4), "unit": unit, "cores": 1,
                            "sample": f"{reps1} {what}", "seconds": round(el1, 2)}}


def oracle_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)


def decode_oracle(sub: wl.Submission, x, weights) -> dict:
    """The oracle, as it stands, over one whole decode submission on the host
    cores: the median of 3 passes on one thread and on every core, as weight
    GB/s (a baseline beside the kernel, not a target)."""
    import oracle
    out = {"kind": "oracle", "passes": 3}
    for key, n in (("all_cores", oracle_threads()), ("single_core", 1)):
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            for j, w in zip(sub.jobs, weights):
                oracle.matmul(x, w, j.fmt, j.n_out, threads=n)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        out[key] = {"cores": n, "ms_median": round(med * 1e3, 4), "gbs": round(sub.weight_bytes / med / 1e9, 4)}
    return out


def stats_device_ms(il, path: str) -> float:
    """Cumulative device time (IL_TIMING=1) of one path from il_stats."""
    for line in il.il_stats().splitlines():
        if line.startswith(path + ":"):
            return float(line.split("device_ms=")[1].split()[0])
    raise RuntimeError(f"no {path} line in il_stats")


def bench_lm_head(args, name: str) -> int:
    """The centroid-masked LM head: one il_centroid_argmax per step (centroid
    logits, top-k, scores of the chosen clusters' tokens, argmax) over
    embedding / centroid copies rotated past the MALL.  It is latency-bound:
    value = bytes it touches (centroids + the gathered embedding rows +
    their ordering entries) per second of wall time."""
    import torch

    import quantized_weight_matmul_amd as il
    h, n_c, k, vocab, t, cfg = wl.LM_HEAD[name]
    per = vocab // n_c
    log(f"[bench] workload {name}: {DESCRIPTIONS[name]}")
    x_np, cen, emb, order = wl.make_lm_head_inputs(name)
    touched = n_c * h * 2 + t * k * per * (h * 2 + 4)
    n_sets = max(1, -(-ROTATE_BYTES // (vocab * h * 2)))
    log(f"[bench] uploading {n_sets} embedding copies x {vocab * h * 2 / 1e6:.1f} MB")
    sets = []
    for _ in range(n_sets):
        pair = (il.il_upload(cen, il.IL_BF16, n_c, h), il.il_upload(emb, il.IL_BF16, vocab, h))
        if None in pair:
            raise RuntimeError(il.il_last_error())
        sets.append(pair)
    x = torch.from_numpy(x_np).cuda()
    od = torch.from_numpy(order.view(np.int32)).cuda()
    tok = torch.empty((t,), dtype=torch.int32, device="cuda")
    ws = torch.empty((il.il_centroid_argmax_workspace(t, n_c, k),), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()  # default priority

    def step(i, s):
        hc, he = sets[i % n_sets]
        if il.il_centroid_argmax(x, t, h, hc, he, od, k, tok, None, None, workspace=ws, stream=s) != 1:
            raise RuntimeError(il.il_last_error())

    ms_per_step, kern_ms, pair_ms = time_steps(step, args, stream, 1)
    value = touched / (ms_per_step * 1e-3) / 1e9
    achieved = touched / (kern_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                "kernel_ms": round(kern_ms, 6),
                "timing": "HIP events on the launch stream around the timed region / calls (3 kernels each)",
                "event_pair_ms_median": round(pair_ms, 6)}
    log(f"[bench] {ms_per_step * 1e3:.2f} us/call wall, {kern_ms * 1e3:.2f} us device ({achieved:.1f} GB/s touched)")
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.centroid_argmax(x_np, cen, emb, order, k)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / reps * (reps + 1) > args.cpu_seconds * 2:
                break
        cpu = {"value": round(touched * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} full oracle LM-head passes ({el / reps * 1e3:.2f} ms each)",
               "seconds": round(el, 2)}
    out = {
        "metric": "centroid-masked LM head: GB/s of bytes touched (latency-bound); us per call in ms_per_step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}", "t": t, "h": h, "centroids": n_c, "top_k": k,
                   "vocab": vocab, "bytes_touched_per_call": touched, "embedding_copies_rotated": n_sets,
                   "timing": "eager" if args.no_graph else "hip-graph"},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_gelu_mul(args, name: str) -> int:
    """The fused gate/up step: one il_matmul_gelu_mul per step over weight
    pairs rotated past the MALL, timed like the matmul workloads (HIP graph,
    events on the launch stream).  The unfused il_matmul of the same pair
    (writing g and u, no GELU) is timed the same way as context."""
    import torch

    import quantized_weight_matmul_amd as il
    fmt, n_out, n_in, t, cfg = wl.GELU_MUL[name]
    log(f"[bench] workload {name}: {DESCRIPTIONS[name]}")
    x_np, G, U = wl.make_gelu_mul_inputs(name)
    per_set = 2 * wl.weight_bytes(fmt, n_out, n_in)
    flops = 4 * t * n_out * n_in
    n_sets = max(1, -(-ROTATE_BYTES // per_set))
    log(f"[bench] uploading {n_sets} gate/up pairs x {per_set / 1e6:.1f} MB")
    sets = []
    for _ in range(n_sets):
        pair = (il.il_upload(G, fmt, n_out, n_in), il.il_upload(U, fmt, n_out, n_in))
        if None in pair:
            raise RuntimeError(il.il_last_error())
        sets.append(pair)
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((t, n_out), dtype=torch.float32, device="cuda")
    g = torch.empty((t, n_out), dtype=torch.float32, device="cuda")
    u = torch.empty((t, n_out), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()  # default priority

    def fused(i, s):
        hg, hu = sets[i % n_sets]
        if il.il_matmul_gelu_mul(x, t, n_in, hg, hu, n_out, y, s) != 1:
            raise RuntimeError(il.il_last_error())

    def unfused(i, s):
        hg, hu = sets[i % n_sets]
        if il.il_matmul(x, t, n_in, [(hg, n_out, g), (hu, n_out, u)], s) != 1:
            raise RuntimeError(il.il_last_error())

    ms_per_step, kern_ms, pair_ms = time_steps(fused, args, stream, 1)
    ms_unfused, kern_unfused, _ = time_steps(unfused, args, stream, 1)
    hbm = t <= STREAMING_MAX_T
    if hbm:
        value, unit = per_set / (ms_per_step * 1e-3) / 1e9, "GB/s"
        achieved, peak = per_set / (kern_ms * 1e-3) / 1e9, HBM_PEAK_GBS
    else:
        value, unit = flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
        achieved, peak = flops / (kern_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS
    roofline = {"bound": "hbm" if hbm else "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(name),
                "kernel_ms": round(kern_ms, 6),
                "timing": "HIP events on the launch stream around the timed region / launches",
                "event_pair_ms_median": round(pair_ms, 6)}
    log(f"[bench] fused {ms_per_step * 1e3:.2f} us/step ({value:.1f} {unit}), kernel {kern_ms * 1e3:.2f} us; "
        f"unfused il_matmul {kern_unfused * 1e3:.2f} us")
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.gelu_mul(x_np, G, U, fmt, n_out, threads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / reps * (reps + 1) > args.cpu_seconds * 2:
                break
        per = el / reps
        cpu = {"value": round((per_set / per / 1e9) if hbm else (flops / per / 1e12), 4), "unit": unit,
               "cores": threads, "kind": "oracle", "sample": f"{reps} full oracle gate/up + GELU passes",
               "seconds": round(el, 2)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": path_dtype([wl.FMT_NAMES[fmt]], t), "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}", "t": t, "n_in": n_in,
                   "jobs": [[wl.FMT_NAMES[fmt], n_out], [wl.FMT_NAMES[fmt], n_out]],
                   "weight_bytes_per_step": per_set, "flops_per_step": flops, "weight_sets_rotated": n_sets,
                   "timing": "eager" if args.no_graph else "hip-graph",
                   "unfused_il_matmul_kernel_ms": round(kern_unfused, 6)},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_quantize(args, name: str) -> int:
    """The upload quantiser: f32 weights resident in HBM -> Q8 / Q4 device
    planes, one il_upload_quantize call per step.  value = f32 input bytes
    per second of whole calls (plane allocation included); the roofline
    takes the quantise kernel alone (HIP events around its launch on the
    library's upload stream, read back through il_stats)."""
    import torch

    import quantized_weight_matmul_amd as il
    os.environ["IL_TIMING"] = "1"
    fmt, n_out, n_in, cfg, tid = wl.QUANTIZE[name]
    n = n_out * n_in
    code_b = n if fmt == wl.Q8 else n // 2
    scale_b = (n // wl.BLOCK) * (4 if fmt == wl.Q8 else 2)
    algo = 4 * n + code_b + 2 * scale_b  # read f32; write codes, scales and their tiled copy
    log(f"[bench] workload {name}: f32 [{n_out}, {n_in}] -> {wl.FMT_NAMES[fmt]} on upload")
    w_np = wl.gen_f32_weight(cfg, tid, n_out, n_in)
    w = torch.from_numpy(w_np).cuda()
    torch.cuda.synchronize()

    def call():
        h = il.il_upload_quantize(w, il.IL_SRC_F32, fmt, n_out, n_in)
        if h is None:
            raise RuntimeError(il.il_last_error())
        return h

    for _ in range(args.warmup):
        call().free()
    steps = args.steps
    dev0 = stats_device_ms(il, "upload_quantize")
    keep, wall = [], 0.0
    for _ in range(steps):
        t0 = time.perf_counter()
        keep.append(call())
        wall += time.perf_counter() - t0
    kern_ms = (stats_device_ms(il, "upload_quantize") - dev0) / steps
    for h in keep:
        h.free()
    ms_per_step = wall * 1e3 / steps
    value = 4 * n / (ms_per_step * 1e-3) / 1e9
    achieved = algo / (kern_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                "kernel_ms": round(kern_ms, 6),
                "timing": "HIP events around each quantise launch on its stream (il_stats device_ms)",
                "algorithmic_bytes_per_launch": algo}
    log(f"[bench] {ms_per_step * 1e3:.1f} us per call ({value:.1f} GB/s of f32 in); kernel "
        f"{kern_ms * 1e3:.2f} us ({achieved:.1f} GB/s algorithmic)")
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        threads = 1  # the oracle quantiser is serial
        rows = max(16, min(n_out, int(2e6 // n_in)))
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.quantize(w_np[:rows], fmt)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / reps * (reps + 1) > args.cpu_seconds * 2:
                break
        cpu = {"value": round(4 * rows * n_in * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "sample": f"{reps} oracle quantisations of the first {rows} rows",
               "seconds": round(el, 2)}
    out = {
        "metric": "quantised GB/s of f32 weights (upload quantiser); roofline on HBM bytes",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: quantise f32 [{n_out}, {n_in}] ~N(0, 0.02) to "
                               f"{wl.FMT_NAMES[fmt]} on upload (input resident in HBM)",
                   "n_out": n_out, "n_in": n_in, "format": wl.FMT_NAMES[fmt]},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# ------------------------------------------------------------ headline line
DECODE_SET = ["c2", "c3a", "c3b", "c4_t1", "c4_t2", "c4_t4", "c4_t8"]
PAGES_DISPATCH_US = 150.0  # Backend::wants doc comment, oxinfer 0.0.0 src/gpu.rs page (Metal)


def host_info() -> dict:
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "oracle_threads": oracle_threads()}


def hip_bus_id() -> str:
    """PCI bus id ("dddd:bb:dd.f") of the HIP device this process uses."""
    import ctypes
    import torch
    lib = ctypes.CDLL("libamdhip64.so")
    buf = ctypes.create_string_buffer(64)
    if lib.hipDeviceGetPCIBusId(buf, 64, torch.cuda.current_device()) != 0:
        raise RuntimeError("hipDeviceGetPCIBusId failed")
    return buf.value.decode().lower()


def _json_of(text: str):
    starts = [i for i in (text.find("{"), text.find("[")) if i >= 0]
    return json.loads(text[min(starts):])


def smi_sample(bus_id: str) -> dict:
    """One `amd-smi metric --clock --power --usage` reading of the GPU with
    this PCI bus id (amd-smi numbers every GPU of the host, not only the ones
    this process sees; the tool's own sampling window; child processes, so
    nothing here touches the GPU): the graphics clock of each XCD, the
    memory clock, power and activity."""
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    try:
        lst = _json_of(subprocess.run([exe, "list", "--json"], capture_output=True, text=True, timeout=30).stdout)
        idx = None
        for e in (lst if isinstance(lst, list) else lst.get("gpu_data", [])):
            if str(e.get("bdf", "")).lower() == bus_id:
                idx = e.get("gpu")
        if idx is None:
            return {"error": f"no amd-smi GPU with bus id {bus_id}", "bus_id": bus_id}
        r = subprocess.run([exe, "metric", "-g", str(idx), "--clock", "--power", "--usage", "--json"],
                           capture_output=True, text=True, timeout=30)
        d = _json_of(r.stdout)
    except (OSError, ValueError, KeyError, AttributeError, subprocess.SubprocessError) as e:
        return {"error": f"{type(e).__name__}: {str(e)[:160]}", "bus_id": bus_id}
    g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)
    out = {"bus_id": bus_id, "amd_smi_gpu": idx, "gfx_mhz": [], "mem_mhz": None, "power": {}, "usage": {}}
    for k, v in (g.get("clock") or {}).items():
        clk = v.get("clk", {}) if isinstance(v, dict) else {}
        val = clk.get("value") if isinstance(clk, dict) else None
        if k.startswith("gfx") and isinstance(val, (int, float)):
            out["gfx_mhz"].append(val)
        elif k.startswith("mem") and isinstance(val, (int, float)):
            out["mem_mhz"] = val
    for part in ("power", "usage"):
        for k, v in (g.get(part) or {}).items():
            if isinstance(v, dict) and isinstance(v.get("value"), (int, float)):
                out[part][k] = [v["value"], v.get("unit")]
    return out


def smi_under_load(bus_id: str, first_after_s: float = 1.5, n: int = 3, gap_s: float = 0.5) -> dict:
    """amd-smi readings taken while the caller keeps the GPU busy: its
    metrics lag the load by about a second, so the first is taken
    first_after_s into the burst, then n - 1 more gap_s apart.  Summary over
    the readings that show the GPU busy (gfx activity >= 90 %): the median
    of their mean XCD clock and of their socket power."""
    time.sleep(first_after_s)
    reads = []
    for i in range(n):
        if i:
            time.sleep(gap_s)
        reads.append(smi_sample(bus_id))
    busy = [r for r in reads if (r.get("usage", {}).get("gfx_activity") or [0])[0] >= 90 and r.get("gfx_mhz")]
    out = {"readings": reads, "busy_readings": len(busy)}
    if busy:
        out["gfx_mhz_median"] = float(np.median([sum(r["gfx_mhz"]) / len(r["gfx_mhz"]) for r in busy]))
        watts = [r["power"]["socket_power"][0] for r in busy if "socket_power" in r.get("power", {})]
        if watts:
            out["socket_power_w_median"] = float(np.median(watts))
    return out


class Rig:
    """One submission set up on the GPU: n_sets weight copies (rotated so a
    rotation exceeds the last-level cache), x and y resident in HBM."""

    def __init__(self, il, sub, x_np, weights, n_sets, cache=None):
        import torch
        self.il, self.sub = il, sub
        self.sets = []
        for k in range(n_sets):
            key = (sub.cfg, sub.n_in, tuple(sub.jobs), k)
            if cache is not None and key in cache:
                self.sets.append(cache[key])
                continue
            hs = [il.il_upload(w, j.fmt, j.n_out, sub.n_in) for w, j in zip(weights, sub.jobs)]
            if any(h is None for h in hs):
                raise RuntimeError(il.il_last_error())
            self.sets.append(hs)
            if cache is not None:
                cache[key] = hs
        self.x = torch.from_numpy(x_np).cuda()
        self.ys = [torch.empty((sub.t, j.n_out), dtype=torch.float32, device="cuda") for j in sub.jobs]

    def step(self, i, s):
        hs = self.sets[i % len(self.sets)]
        jobs = [(h, j.n_out, y) for h, j, y in zip(hs, self.sub.jobs, self.ys)]
        if self.il.il_matmul(self.x, self.sub.t, self.sub.n_in, jobs, s) != 1:
            raise RuntimeError(self.il.il_last_error())


def time_eager(step, steps: int, warmup: int, stream):
    """K eager calls bracketed by synchronisations: (wall ms per call, device
    ms per call from HIP events on the launch stream around the burst)."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(steps):
            step(i, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, e0.elapsed_time(e1) / steps


def time_graph(step, steps: int, warmup: int, stream, settle=None):
    """K calls captured in one HIP graph and replayed: (wall ms per call,
    device ms per call from HIP events around the replay).  settle: untimed
    work run right before the timed replay."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream, capture_error_mode="relaxed"):
        for i in range(steps):
            step(i, torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    if settle:
        settle()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    return wall * 1e3 / steps, e0.elapsed_time(e1) / steps


FLUSH_BYTES = 512 << 20  # > the 256 MiB last-level cache


def prefill_kernel_split(il, step, calls: int, stream):
    """Device time of the x -> bf16 pre-pass and of the GEMM launch in each of
    `calls` eager calls, from HIP events the library records on the launch
    stream around each of them (IL_TIMING=1, which waits for every call).  A
    512 MiB write (a fill kernel, outside the timed kernels) runs before each
    call, so neither kernel finds the previous call's x, bf16 x or y in the
    last-level cache.  Returns (GEMM ms, pre-pass ms) lists, one entry a call."""
    import torch
    scratch = torch.empty((FLUSH_BYTES,), dtype=torch.uint8, device="cuda")

    def read():
        for line in il.il_stats().splitlines():
            if line.startswith("prefill_gemm:"):
                f = dict(kv.split("=") for kv in line.split(":", 1)[1].split())
                return float(f["device_ms"]), float(f["prepass_ms"]), int(f["split_calls"])
        raise RuntimeError("no prefill_gemm line in il_stats")

    gemm, pre = [], []
    os.environ["IL_TIMING"] = "1"
    try:
        with torch.cuda.stream(stream):
            for i in range(calls):
                scratch.fill_(i & 0xFF)
                d0, p0, n0 = read()
                step(i, stream)
                d1, p1, n1 = read()
                if n1 - n0 != 1:
                    raise RuntimeError("a timed prefill call was not split into pre-pass and GEMM")
                pre.append(p1 - p0)
                gemm.append(d1 - d0 - (p1 - p0))
        torch.cuda.synchronize()
    finally:
        del os.environ["IL_TIMING"]
    return gemm, pre


def spread(v) -> dict:
    """median / p10 / p90 / mean (ms) of per-call times."""
    q = sorted(v)
    at = lambda f: q[min(len(q) - 1, int(f * len(q)))]
    return {"median": round(statistics.median(q), 6), "p10": round(at(0.1), 6), "p90": round(at(0.9), 6),
            "mean": round(sum(q) / len(q), 6), "calls": len(q)}


def input_digests(sub, x_np, weights) -> dict:
    import hashlib
    h = lambda a: hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]
    d = {"x": h(x_np)}
    for j, w in zip(sub.jobs, weights):
        d[f"w{j.tensor_id}"] = h(w)
    return d


def decode_entry(il, name: str, args, stream, cache) -> dict:
    sub = wl.SUBMISSIONS[name]
    x_np = wl.make_x(sub)
    weights = wl.make_weights(sub)
    n_sets = max(1, -(-ROTATE_BYTES // sub.weight_bytes))
    rig = Rig(il, sub, x_np, weights, n_sets, cache)
    steps = max(200, args.steps)
    wall_g, dev_g = time_graph(rig.step, steps, 20, stream)
    wall_e, _ = time_eager(rig.step, steps, 20, stream)
    launches = len({j.fmt for j in sub.jobs})
    achieved = sub.weight_bytes / (dev_g * 1e-3) / 1e9
    e = {"workload": DESCRIPTIONS[name], "t": sub.t, "weight_bytes": sub.weight_bytes,
         "kernel_ms": round(dev_g / launches, 6), "launches_per_call": launches,
         "achieved_gbs": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBS, 4),
         "traffic": measured_traffic(name), "graph_us_per_call": round(wall_g * 1e3, 3),
         "eager_us_per_call": round(wall_e * 1e3, 3), "weight_sets_rotated": n_sets,
         "dtype": path_dtype([wl.FMT_NAMES[j.fmt] for j in sub.jobs], sub.t),
         "input_sha256_16": input_digests(sub, x_np, weights)}
    log(f"[bench] {name}: kernel {e['kernel_ms'] * 1e3:.2f} us ({achieved:.0f} GB/s, {e['frac']:.3f} of HBM), "
        f"graph {e['graph_us_per_call']:.2f} us/call, eager {e['eager_us_per_call']:.2f} us/call")
    del rig
    if args.cpu_seconds > 0:
        e["oracle"] = decode_oracle(sub, x_np, weights)
        e["oracle"]["kernel_over_all_cores"] = round(achieved / e["oracle"]["all_cores"]["gbs"], 1)
    return e


def wants_calibration(il, stream, cpu) -> dict:
    """The il_wants threshold from measurements: the work the host oracle
    does in the time one launch-bound call takes (eager calls of the smallest
    configuration, bf16 [1024, 256] at t = 1, host validation and launch
    included).  A call of fewer flops than that would finish sooner on the
    host; il_wants should say yes above it.  Also whether the calibrated
    threshold says yes to every configuration."""
    sub = wl.SUBMISSIONS["c1"]
    x_np, weights = wl.make_x(sub), wl.make_weights(sub)
    rig = Rig(il, sub, x_np, weights, 1)
    wall_ms, _ = time_eager(rig.step, 2000, 200, stream)
    del rig
    out = {"tiny_call_us": round(wall_ms * 1e3, 3), "default_min_flop": 262144}
    if cpu is None:
        return out
    out["c1_oracle"] = decode_oracle(sub, x_np, weights)
    flops_per_s = cpu["value"] * 1e12  # the oracle on every host core (prefill sample)
    min_flop = wall_ms * 1e-3 * flops_per_s
    old = os.environ.get("IL_WANTS_MIN_FLOP")
    os.environ["IL_WANTS_MIN_FLOP"] = repr(min_flop)
    try:
        says = {n: all(il.il_wants(j.n_out, s.n_in, s.t) == 1 for j in s.jobs) for n, s in wl.SUBMISSIONS.items()}
    finally:
        if old is None:
            del os.environ["IL_WANTS_MIN_FLOP"]
        else:
            os.environ["IL_WANTS_MIN_FLOP"] = old
    out.update({"oracle_tflops_all_cores": cpu["value"], "calibrated_min_flop": round(min_flop),
                "calibrated_over_default": round(min_flop / 262144, 3),
                "yes_for_every_config": all(says.values()),
                "no_for": sorted(n for n, v in says.items() if not v)})
    log(f"[bench] il_wants: a launch-bound call takes {out['tiny_call_us']} us, in which the oracle does "
        f"{min_flop:.3g} flop (default threshold 2^18 = 262144); yes for every config: {out['yes_for_every_config']}")
    return out


def bench_headline(args) -> int:
    """The default line: the bf16 prefill (2048 tokens through [4096 | 14336]
    x 4096, the largest configuration that fits one GPU) as TFLOP/s, with the
    decode workloads' weight GB/s in a `decode` object beside it."""
    import torch

    import quantized_weight_matmul_amd as il
    name = "c5a"
    sub = wl.SUBMISSIONS[name]
    log(f"[bench] headline workload {name}: {DESCRIPTIONS[name]}")
    x_np = wl.make_x(sub)
    weights = wl.make_weights(sub)
    n_sets = max(1, -(-ROTATE_BYTES // sub.weight_bytes))
    log(f"[bench] uploading {n_sets} weight sets x {sub.weight_bytes / 1e6:.1f} MB")
    rig = Rig(il, sub, x_np, weights, n_sets)
    stream = torch.cuda.Stream()  # default priority

    # Calls right after an idle spell run at boost clocks; back-to-back calls
    # settle lower (the first GEMMs of a burst measured ~296 us, later ones
    # 330-375 us).  Each timed section therefore follows `settle` seconds of
    # untimed calls, so the figures are the sustained rate.
    def burst(seconds, sync=True):
        def run():
            calls = max(1, int(seconds / 3e-4))
            with torch.cuda.stream(stream):
                for i in range(calls):
                    rig.step(i, stream)
            if sync:
                torch.cuda.synchronize()
        return run

    # There is no live shader-clock reading in the kernels: s_memtime counts
    # ~2.4 GHz whatever the load.  The GEMM's own counters bound it
    # (SQ_BUSY_CYCLES per shader array over the kernel's duration; see the
    # committed profile of this workload), and amd-smi is read once while
    # back-to-back calls keep the GPU busy (its own averaging window).
    clock = {"live_mhz": None, "max_engine_mhz": 2400,
             "note": "not read in the kernels; SQ_BUSY_CYCLES / 32 shader arrays over the GEMM's duration bounds "
                     "it, profiles/gemm_bf16_prefill_2048x18432x4096.txt; smi_under_load: one amd-smi reading "
                     "series of this process's GPU (matched by PCI bus id) taken while bursts of these calls run "
                     "(its metrics lag the load by about a second); the roofline keeps the published peak"}
    smi = {}
    try:
        bus = hip_bus_id()
    except (OSError, RuntimeError, AttributeError) as e:
        bus = f"unknown ({type(e).__name__})"
    sampler = threading.Thread(target=lambda: smi.update(smi_under_load(bus)), daemon=True)
    sampler.start()
    t_end = time.perf_counter() + 30.0
    while sampler.is_alive() and time.perf_counter() < t_end:
        burst(0.5)()  # keep the GPU on this workload while the tool samples
    sampler.join(timeout=1.0)
    clock["smi_under_load"] = smi or {"error": "no reading within 30 s"}
    log(f"[bench] amd-smi during the calls: {clock['smi_under_load'].get('busy_readings')} busy readings, "
        f"gfx {clock['smi_under_load'].get('gfx_mhz_median')} MHz, "
        f"{clock['smi_under_load'].get('socket_power_w_median')} W")
    burst(args.settle)()
    # ---- timed region: K eager calls (host validation and launches included) ----
    ms_per_step, dev_ms = time_eager(rig.step, args.steps, args.warmup, stream)
    burst(args.settle / 3)()
    gemm_calls, pre_calls = prefill_kernel_split(il, rig.step, max(20, min(args.steps, 100)), stream)
    gemm_ms, pre_ms = statistics.median(gemm_calls), statistics.median(pre_calls)
    wall_g, dev_g = time_graph(rig.step, args.steps, args.warmup, stream, settle=burst(args.settle / 3))
    value = sub.flops / (ms_per_step * 1e-3) / 1e12
    achieved = sub.flops / (gemm_ms * 1e-3) / 1e12
    log(f"[bench] {ms_per_step * 1e3:.1f} us/call eager ({value:.1f} TFLOP/s), graph {wall_g * 1e3:.1f} us/call; "
        f"GEMM kernel {gemm_ms * 1e3:.1f} us ({achieved:.1f} TFLOP/s), pre-pass {pre_ms * 1e3:.1f} us")
    digests = input_digests(sub, x_np, weights)
    del rig

    decode = {}
    if not args.no_decode:
        cache = {}
        for dn in DECODE_SET:
            decode[dn] = decode_entry(il, dn, args, stream, cache)
        cache.clear()

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] oracle on the host cores for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(sub, x_np, weights, args.cpu_seconds)
    wants = wants_calibration(il, stream, cpu)

    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(name, "gemm_bf16_kernel"),
                "kernel": "gemm_bf16_kernel", "kernel_ms": round(gemm_ms, 6), "prepass_ms": round(pre_ms, 6),
                "kernel_ms_per_call": spread(gemm_calls), "prepass_ms_per_call": spread(pre_calls),
                "call_device_ms": round(dev_ms, 6),
                "call_frac": round(sub.flops / (dev_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "timing": "kernel_ms / prepass_ms: medians over eager calls of the HIP events the library "
                          "records on the launch stream around each of the call's two kernels (IL_TIMING=1), "
                          "with a 512 MiB scratch write before each call; call_device_ms: HIP events on the "
                          "launch stream around the timed burst / calls"}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}", "t": sub.t, "n_in": sub.n_in,
                   "jobs": [[wl.FMT_NAMES[j.fmt], j.n_out] for j in sub.jobs],
                   "weight_bytes_per_step": sub.weight_bytes, "flops_per_step": sub.flops,
                   "weight_sets_rotated": n_sets,
                   "timing": "eager il_matmul calls, host validation and launches included",
                   "eager_us_per_call": round(ms_per_step * 1e3, 3),
                   "graph_us_per_call": round(wall_g * 1e3, 3),
                   "pages_dispatch_cost_us": PAGES_DISPATCH_US,
                   "input_sha256_16": digests, "host": host_info(), "shader_clock": clock,
                   "il_wants": wants},
        "roofline": roofline, "cpu_baseline": cpu, "decode": decode,
    }
    print(json.dumps(out), flush=True)
    return 0


# Decode shapes of model-like layers for the dispatch sweep: (format, n_out
# of each job, n_in).
SWEEP_SHAPES = [(wl.Q4, [17408, 17408], 5120), (wl.Q4, [4096, 1024, 1024], 4096), (wl.Q4, [4096], 14336),
                (wl.Q4, [1024], 4096), (wl.Q8, [14336, 14336], 4096), (wl.Q8, [4096], 14336),
                (wl.Q8, [1024, 1024], 4096)]


def decode_sweep(args) -> int:
    """Both decode kernel families (IL_DECODE=valu / mfma) and the library's
    own choice over model-like shapes at t = 1, 2, 4, 8: device us per call
    (HIP events around a burst of eager calls, weights rotated past the
    last-level cache); one JSON line."""
    import torch

    import quantized_weight_matmul_amd as il
    stream = torch.cuda.Stream()  # default priority
    rows = []
    for fmt, n_outs, n_in in SWEEP_SHAPES:
        ws = [wl.gen_weight(fmt, 90, j, n, n_in) for j, n in enumerate(n_outs)]
        bytes_set = sum(int(w.nbytes) for w in ws)
        n_sets = max(1, -(-ROTATE_BYTES // bytes_set))
        sets = [[il.il_upload(w, fmt, n, n_in) for w, n in zip(ws, n_outs)] for _ in range(n_sets)]
        if any(h is None for hs in sets for h in hs):
            raise RuntimeError(il.il_last_error())
        for t in (1, 2, 4, 8):
            x = torch.from_numpy(np.random.default_rng(t).standard_normal((t, n_in)).astype(np.float32)).cuda()
            ys = [torch.empty(t, n, device="cuda") for n in n_outs]

            def step(i, s):
                hs = sets[i % n_sets]
                if il.il_matmul(x, t, n_in, [(h, n, y) for h, n, y in zip(hs, n_outs, ys)], stream=s) != 1:
                    raise RuntimeError(il.il_last_error())
            row = {"fmt": wl.FMT_NAMES[fmt], "n_outs": n_outs, "n_in": n_in, "t": t}
            for mode in ("valu", "mfma", "auto"):
                if mode == "auto":
                    os.environ.pop("IL_DECODE", None)
                else:
                    os.environ["IL_DECODE"] = mode
                _, dev_ms = time_eager(step, args.steps, args.warmup, stream)
                row[f"{mode}_us"] = round(dev_ms * 1e3, 2)
            os.environ.pop("IL_DECODE", None)
            row["auto_is_faster_family"] = row["auto_us"] <= 1.05 * min(row["valu_us"], row["mfma_us"])
            log(f"[sweep] {row['fmt']} {n_outs} x {n_in} t={t}: streaming {row['valu_us']} us, matrix-core "
                f"{row['mfma_us']} us, dispatch {row['auto_us']} us")
            rows.append(row)
        for hs in sets:
            for h in hs:
                il.il_free(h)
    print(json.dumps({"metric": "decode kernel dispatch sweep", "unit": "device us per call", "steps": args.steps,
                      "rows": rows}), flush=True)
    return 0


def calibrate_read(sizes_mb) -> int:
    """The read ceiling: il_read_probe (a plain streaming read, no arithmetic)
    over buffers of the given sizes, rotated so that one rotation exceeds
    1 GiB, in a sweep of launch shapes; prints one JSON line with the best
    shape and rate per size."""
    import torch

    import quantized_weight_matmul_amd as il
    stream = torch.cuda.Stream()
    out = {"metric": "plain streaming read GB/s (il_read_probe), best launch shape per size",
           "unit": "GB/s", "peak": HBM_PEAK_GBS, "sizes": {}}
    for mb in sizes_mb:
        nbytes = int(mb * 1e6) // 16 * 16
        n_bufs = max(1, -(-ROTATE_BYTES // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(k) for k in range(n_bufs)]
        sink = torch.empty(nbytes // 1024 + 1, dtype=torch.int32, device="cuda")
        rows = []
        for waves in (4, 8, 16):
            for chunk_kib in (16, 32, 64, 128, 256):
                chunk = chunk_kib * 1024
                for depth in (2, 4, 8):
                    if chunk < 64 * waves * 16 * depth:
                        continue  # fewer bytes than one round of the ring
                    def launch(i, s):
                        if il.il_read_probe(bufs[i % n_bufs], nbytes, chunk, waves, depth, sink,
                                            sink.numel() * 4, s) != 1:
                            raise RuntimeError(il.il_last_error())
                    _, dev_ms = time_eager(launch, 40, 8, stream)
                    gbs = nbytes / (dev_ms * 1e-3) / 1e9
                    rows.append({"waves": waves, "chunk_kib": chunk_kib, "depth": depth,
                                 "workgroups": -(-nbytes // chunk), "us": round(dev_ms * 1e3, 2),
                                 "gbs": round(gbs, 1)})
        rows.sort(key=lambda r: -r["gbs"])
        best = rows[0]
        log(f"[read] {mb} MB: best {best['gbs']:.0f} GB/s ({best['gbs'] / HBM_PEAK_GBS:.3f} of peak) with "
            f"{best['waves']} waves x {best['chunk_kib']} KiB, depth {best['depth']} ({best['us']} us); "
            f"next {[(r['waves'], r['chunk_kib'], r['depth'], r['gbs']) for r in rows[1:4]]}")
        out["sizes"][f"{mb}MB"] = {"bytes": nbytes, "buffers_rotated": n_bufs, "best": best,
                                   "frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4), "top5": rows[:5]}
        del bufs
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    choices=sorted(wl.SUBMISSIONS) + sorted(wl.QUANTIZE) + sorted(wl.GELU_MUL) + sorted(wl.LM_HEAD),
                    help="time one workload alone (default: the headline line, bf16 prefill c5a with the "
                         "decode workloads beside it)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget (0: skip)")
    ap.add_argument("--no-graph", action="store_true", help="single workload: time eager launches, not a graph")
    ap.add_argument("--no-decode", action="store_true", help="headline line without the decode object")
    ap.add_argument("--settle", type=float, default=1.5,
                    help="headline: seconds of untimed calls before the timed sections (sustained clocks)")
    ap.add_argument("--calibrate-read", default="", metavar="MB[,MB...]",
                    help="only time a plain streaming read (il_read_probe) of buffers of these sizes in a "
                         "sweep of launch shapes: the read ceiling of the decode kernels")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="only time both decode kernel families and the dispatch's choice over model-like shapes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty(n, device="cuda")
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calibrate_copy} MiB five times")
        return 0

    if args.calibrate_read:
        return calibrate_read([float(v) for v in args.calibrate_read.split(",")])
    if args.decode_sweep:
        return decode_sweep(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run it with --gpus 1.", file=sys.stderr)
        return 2
    import torch

    import quantized_weight_matmul_amd as il

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.workload is None:
        return bench_headline(args)
    if args.workload in wl.QUANTIZE:
        return bench_quantize(args, args.workload)
    if args.workload in wl.GELU_MUL:
        return bench_gelu_mul(args, args.workload)
    if args.workload in wl.LM_HEAD:
        return bench_lm_head(args, args.workload)
    sub = wl.SUBMISSIONS[args.workload]
    streaming = sub.t <= STREAMING_MAX_T
    log(f"[bench] workload {sub.name}: {DESCRIPTIONS[sub.name]}")
    x_np = wl.make_x(sub)
    weights = wl.make_weights(sub)
    per_set = sub.weight_bytes
    n_sets = max(1, -(-ROTATE_BYTES // per_set)) if streaming else max(2, -(-ROTATE_BYTES // per_set))
    log(f"[bench] uploading {n_sets} weight sets x {per_set / 1e6:.1f} MB")
    rig = Rig(il, sub, x_np, weights, n_sets)
    stream = torch.cuda.Stream()  # default priority
    ms_per_step, kern_ms, pair_ms = time_steps(rig.step, args, stream, len({j.fmt for j in sub.jobs}))
    return report(args, sub, per_set, n_sets, ms_per_step, kern_ms, pair_ms, x_np, weights)


def time_steps(step, args, stream, launches_per_step):
    """Warm-up, event pairs around a few eager launches, then K steps in one
    HIP graph (or eager) with HIP events on the launch stream around them.
    Returns (wall ms per step, kernel ms per launch, median event pair ms)."""
    import torch
    n_ev = min(args.steps, 100)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i, stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_ev)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            step(i, stream)
            b.record(stream)
    torch.cuda.synchronize()
    pair_ms = float(np.median([a.elapsed_time(b) for a, b in evs]))

    # ---- timed region: K steps; HIP events on the kernels' stream around it ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(args.steps):
                step(i, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        total_s = time.perf_counter() - t0
    else:
        g_warm = torch.cuda.CUDAGraph()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream, capture_error_mode="relaxed"):
            for i in range(args.warmup):
                step(i, torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=stream, capture_error_mode="relaxed"):
            for i in range(args.steps):
                step(i, torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        total_s = time.perf_counter() - t0
    ms_per_step = total_s * 1e3 / args.steps
    kern_ms = e0.elapsed_time(e1) / (args.steps * launches_per_step)
    return ms_per_step, kern_ms, pair_ms


def report(args, sub, per_set, n_sets, ms_per_step, kern_ms, pair_ms, x_np, weights) -> int:
    decode = sub.t <= 8
    streaming = sub.t <= STREAMING_MAX_T
    launches_per_step = len({j.fmt for j in sub.jobs})
    if streaming:
        value = per_set / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = per_set / launches_per_step / (kern_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        value = sub.flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = sub.flops / launches_per_step / (kern_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "the whole call (x -> bf16 pre-pass and GEMM)"}
    roofline["traffic"] = measured_traffic(sub.name)
    roofline["kernel_ms"] = round(kern_ms, 6)
    roofline["timing"] = "HIP events on the launch stream around the timed region / launches"
    roofline["event_pair_ms_median"] = round(pair_ms, 6)
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step, {value:.1f} {unit}; kernel {kern_ms * 1e3:.2f} us "
        f"({achieved:.1f} {unit}); single-launch event pair {pair_ms * 1e3:.2f} us")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] oracle on the host cores for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(sub, x_np, weights, args.cpu_seconds)

    fmts = sorted({wl.FMT_NAMES[j.fmt] for j in sub.jobs})
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype([wl.FMT_NAMES[j.fmt] for j in sub.jobs], sub.t),
        "data": "synthetic",
        "config": {
            "workload": f"{sub.name}: {DESCRIPTIONS[sub.name]}",
            "t": sub.t,
            "n_in": sub.n_in,
            "jobs": [[wl.FMT_NAMES[j.fmt], j.n_out] for j in sub.jobs],
            "weight_formats": fmts,
            "weight_bytes_per_step": per_set,
            "flops_per_step": sub.flops,
            "weight_sets_rotated": n_sets,
            "timing": "eager" if args.no_graph else "hip-graph",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
