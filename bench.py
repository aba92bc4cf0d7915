#!/usr/bin/env python3
"""Benchmark of the fused row softmax on one MI355X.

A step is one launch of the library's softmax over one whole input matrix
(the full hot path: load, max, exp, sum, normalise, store).  The headline
workload is 8192 x 4096 fp16 (the shape whose bandwidth the
"fused-softmax-roofline" page reports); the other fixed shapes are timed the
same way and reported under "shapes".  Metric: achieved HBM bandwidth
2 * rows * cols * sizeof / time, and its fraction of MI355X's 8 TB/s.

Timing: inputs are resident in HBM before the timed region; R input/output
buffer pairs (R * pair >= 1 GiB) rotate so the 256 MB Infinity Cache cannot
serve them; W untimed launches, then K launches between two HIP events on the
launch stream, with a device synchronisation on both sides.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-cpu]
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from row_wise_softmax_amd import binding  # noqa: E402
from row_wise_softmax_amd import workloads as W  # noqa: E402

METRIC = "achieved HBM GB/s (2·rows·cols·bytes/time) and % of MI355X peak, per shape"
# The pages' own figure for the same metric and shape: 8192 x 4096 fp16 at about
# 2.8 TB/s (134.2 MB in 48 us) on an H100 ("fused-softmax-roofline", its
# results).  Another machine's number: vs_baseline is context, not a target.
PAGES_GBPS = 2800.0
PEAK_GBPS = 8000.0
HEADLINE = "c3"
FIXED = ["c1", "c2", "c3", "c4"]
ROTATE_BYTES = 1 << 30
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def upload(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(x) if dtype == "f32" else torch.from_numpy(x.view(np.int16)).view(torch_dtype(dtype))
    return t.to("cuda")


def n_buffers(pair_bytes: int) -> int:
    return max(2, -(-ROTATE_BYTES // pair_bytes))


SPIN_S = 0.3  # untimed launches before each measurement, for steady clocks


def spin_up(launch, n_buf: int, seconds: float) -> None:
    """Launch repeatedly for `seconds` (untimed): from idle the GPU needs a few
    hundred milliseconds of load to reach its steady clocks, and a few
    milliseconds of warm-up measure the ramp instead of the kernel (3% on the
    fp16 softmax, up to 25% on attention)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            launch(i % n_buf)
            i += 1
        torch.cuda.synchronize()


def time_launches(launch, n_buf: int, steps: int, warmup: int, spin_s: float = SPIN_S) -> float:
    """Mean ms per launch over `steps` launches, cycling buffer index 0..n_buf-1,
    after a spin-up of `spin_s` seconds and `warmup` untimed launches."""
    import torch
    stream = torch.cuda.current_stream()
    if spin_s > 0:
        spin_up(launch, n_buf, spin_s)
    for i in range(warmup):
        launch(i % n_buf)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i % n_buf)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def time_graph(res, n_launch: int, replays: int = 5) -> float:
    """Mean ms per launch when `n_launch` softmax launches (cycling the buffer
    sets) are captured in one HIP graph and the graph is replayed: the same
    kernels without the host's per-launch cost, which bounds the eager rate of
    launches a few microseconds long."""
    import torch
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    eager_stream = res.stream
    try:
        res.stream = side.cuda_stream
        with torch.cuda.stream(side):  # warm-up off the capture, as torch asks
            for i in range(3):
                res.softmax(i % res.n)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            res.stream = torch.cuda.current_stream().cuda_stream
            for i in range(n_launch):
                res.softmax(i % res.n)
    finally:
        res.stream = eager_stream
    torch.cuda.synchronize()
    graph.replay()  # untimed
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    start.record(stream)
    for _ in range(replays):
        graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (replays * n_launch)
    graph.reset()
    return ms


class Resident:
    """R copies of one input in HBM plus R outputs."""

    def __init__(self, wl: W.Workload, x: np.ndarray | None = None):
        import torch
        self.wl = wl
        x = wl.generate() if x is None else x
        self.x_host = x
        pair = 2 * x.nbytes
        self.n = n_buffers(pair)
        first = upload(x, wl.dtype)
        self.ins = [first] + [first.clone() for _ in range(self.n - 1)]
        self.outs = [torch.empty_like(first) for _ in range(self.n)]
        self.code = W.dtype_code(wl.dtype)
        self.stream = torch.cuda.current_stream().cuda_stream

    def softmax(self, i: int, kernel_id: int | None = None) -> None:
        wl = self.wl
        if kernel_id is None:
            binding.softmax_fwd(self.ins[i].data_ptr(), self.outs[i].data_ptr(), wl.rows, wl.cols, wl.cols,
                                self.code, self.stream)
        else:
            binding.softmax_fwd_kernel(kernel_id, self.ins[i].data_ptr(), self.outs[i].data_ptr(), wl.rows,
                                       wl.cols, wl.cols, self.code, self.stream)

    def copy(self, i: int) -> None:
        binding.bench_copy(self.ins[i].data_ptr(), self.outs[i].data_ptr(), self.x_host.nbytes, self.stream)

    def memcpy(self, i: int) -> None:
        self.outs[i].copy_(self.ins[i])

    def output(self, i: int = 0) -> np.ndarray:
        import torch
        o = self.outs[i].cpu()
        return o.numpy() if self.wl.dtype == "f32" else o.view(torch.int16).numpy().view(np.uint16)


def causal_c2(steps: int, warmup: int) -> dict:
    """c2's structure with the mask and scale fused into the kernel: raw q k^T
    scores in, softmax(scores / 8) with columns j > i masked out.  The kernel
    reads only the kept columns (about half) and writes every column."""
    import torch
    wl = W.WORKLOADS["c2"]
    rng = np.random.default_rng(list(wl.seed))
    q = rng.standard_normal((wl.cols, 64))
    k = rng.standard_normal((wl.cols, 64))
    x = W.cast(q @ k.T, "f32")
    res = Resident(wl, x=x)
    stream = res.stream

    def launch(i):
        binding.softmax_fwd_causal(res.ins[i].data_ptr(), res.outs[i].data_ptr(), wl.rows, wl.cols, wl.cols,
                                   0.125, 0, res.code, stream)

    ms = time_launches(launch, res.n, steps, warmup)
    n = wl.rows
    actual = (n * (n + 1) // 2 + n * wl.cols) * 4  # kept columns read + every column written
    kid = binding.softmax_select(res.ins[0].data_ptr(), res.outs[0].data_ptr(), wl.cols, wl.cols, res.code,
                                 rows=wl.rows, causal=True)
    d = {"workload": "c2_causal_2048x2048_f32_fused_mask_scale", "rows": n, "cols": wl.cols, "dtype": "f32",
         "kernel": binding.kernel_table()[kid].name, "buffers": res.n, "us": round(ms * 1e3, 3),
         "gbps": round(wl.bytes / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(wl.bytes / (ms * 1e-3) / 1e9 / PEAK_GBPS, 4),
         "actual_bytes": actual, "actual_gbps": round(actual / (ms * 1e-3) / 1e9, 1),
         "note": "gbps uses the metric's 2*rows*cols*4 bytes; actual_gbps the bytes moved (masked inputs are not read)"}
    log(f"[bench] {d['workload']}: {d['us']} us  metric {d['gbps']} GB/s  actual {d['actual_gbps']} GB/s  kernel={d['kernel']}")
    del res
    torch.cuda.synchronize()
    return d


def split_shapes(steps: int, warmup: int) -> dict:
    """Few, wide rows: softmax_fwd (which splits them through its output), the
    width's one-workgroup-per-row kernel forced, and softmax_fwd_split with a
    caller workspace."""
    import torch
    out = {}
    for key in ("wide_f32", "wide_bf16"):
        wl = W.WORKLOADS[key]
        res = Resident(wl)
        nbytes = binding.split_workspace_bytes(wl.rows, wl.cols, res.code)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        fwd = time_launches(res.softmax, res.n, steps, warmup)
        variant, block = binding.softmax_select_variant(wl.cols, res.code)
        one = time_launches(lambda i: binding.softmax_fwd_variant(res.ins[i].data_ptr(), res.outs[i].data_ptr(),
                                                                   wl.rows, wl.cols, wl.cols, res.code, variant, block,
                                                                   res.stream), res.n, steps, warmup)
        spl = time_launches(lambda i: binding.softmax_fwd_split(res.ins[i].data_ptr(), res.outs[i].data_ptr(), wl.rows,
                                                                 wl.cols, wl.cols, res.code, ws.data_ptr(), nbytes, 1,
                                                                 res.stream), res.n, steps, warmup)
        rate = lambda ms: round(wl.bytes / (ms * 1e-3) / 1e9, 1)
        d = {"workload": wl.name, "rows": wl.rows, "cols": wl.cols, "dtype": wl.dtype,
             "kernel": kernel_name(res), "us": round(fwd * 1e3, 3), "gbps": rate(fwd),
             "one_wg_per_row": {"variant": variant, "block": block, "us": round(one * 1e3, 3), "gbps": rate(one)},
             "split_workspace": {"us": round(spl * 1e3, 3), "gbps": rate(spl)},
             "note": "gbps by the metric's 2*rows*cols*size bytes; softmax_fwd splits these rows with the tile pairs "
                     "kept in its output (three kernels, two for calls of up to 1024 tiles), softmax_fwd_split with a "
                     "workspace (two); in the counter runs "
                     "(profiles/counters_wide_rows.txt) the split moved 1.5x those bytes, one workgroup per row 1.0x"}
        log(f"[bench] {wl.name}: softmax_fwd {d['us']} us ({d['gbps']} GB/s, {d['kernel']})"
            f"  one wg per row {d['one_wg_per_row']['us']} us  split+workspace {d['split_workspace']['us']} us")
        out[key] = d
        del res, ws
    torch.cuda.synchronize()
    return out


def attention_shapes(steps: int, warmup: int) -> dict:
    """Fused attention forward (MFMA) on the shapes of the attention page's
    table: batch 4, 32 heads, head dim 128, causal, context 1024 ... 32768,
    seeded N(0, 1) inputs drawn on the device."""
    import torch
    out = {}
    # the context lengths of the attention page's table (fp16), and bf16 at 4096
    for dt, n in (("f16", 1024), ("f16", 4096), ("f16", 8192), ("f16", 16384), ("f16", 32768), ("bf16", 4096)):
        b, h, d = 4, 32, 128
        g = torch.Generator(device="cuda").manual_seed(7)  # drawn on the device: up to 3 GB of inputs
        tdt = torch_dtype(dt)
        qkv = [torch.randn((b, h, n, d), generator=g, device="cuda", dtype=torch.float32).to(tdt) for _ in range(3)]
        o = torch.empty_like(qkv[0])
        stream = torch.cuda.current_stream().cuda_stream
        code = W.dtype_code(dt)

        def launch(i):
            binding.attention_fwd(qkv[0].data_ptr(), qkv[1].data_ptr(), qkv[2].data_ptr(), o.data_ptr(), b, h, n, n, d,
                                  1.0 / d ** 0.5, True, code, stream)

        reps = max(3, min(steps, 20 if n <= 8192 else 5))
        ms = time_launches(launch, 1, reps, max(1, min(warmup, 3)))
        flops = 4.0 * b * h * d * (n * (n + 1) / 2)  # two products over the kept (causal) keys
        nbytes = 4.0 * b * h * n * d * 2  # Q, K, V read once and O written once
        tf = flops / (ms * 1e-3) / 1e12
        bound_us = max(flops / 2.5e15, nbytes / (PEAK_GBPS * 1e9)) * 1e6  # the slower of MFMA and HBM at peak
        key = f"attention_{dt}_b{b}_h{h}_n{n}_d{d}_causal"
        out[key] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / 2500.0, 4),
                    "bound": "mfma" if flops / 2.5e15 >= nbytes / (PEAK_GBPS * 1e9) else "hbm",
                    "roofline_us": round(bound_us, 1), "frac_of_roofline": round(bound_us / (ms * 1e3), 4),
                    "note": "flops = 4*b*h*d*n(n+1)/2 (kept keys only); bytes = 8*b*h*n*d (Q, K, V in, O out); "
                            "roofline = max(flops / 2.5 PFLOP/s dense fp16/bf16 MFMA, bytes / 8 TB/s)"}
        log(f"[bench] {key}: {out[key]['us']} us  {out[key]['tflops']} TFLOP/s ({100 * out[key]['frac_of_mfma_peak']:.1f}% of MFMA"
            f" peak; {out[key]['bound']}-bound roofline {out[key]['roofline_us']} us, {100 * out[key]['frac_of_roofline']:.1f}%)")
        del qkv, o
    torch.cuda.synchronize()
    return out


def kernel_name(res: Resident) -> str:
    kid = binding.softmax_select(res.ins[0].data_ptr(), res.outs[0].data_ptr(), res.wl.cols, res.wl.cols,
                                 res.code, rows=res.wl.rows)
    if kid == binding.SPLIT_KERNEL:
        return f"split_{res.wl.dtype}_via_out"
    return binding.kernel_table()[kid].name


def measure_shape(key: str, steps: int, warmup: int, with_copy: bool, with_unfused: bool = False,
                  light: bool = False, oracle_timing: bool = True) -> dict:
    """One shape: the dispatch pick timed over rotating buffers, and (with_copy) the
    same-size copy kernel.  `light` skips the memcpy, graph and warm-cache figures
    (the width sweep's 24 tensors); `oracle_timing` adds the single-threaded
    oracle's rate on the same input (the whole input, or a bounded row sample)."""
    wl = W.WORKLOADS[key]
    log(f"[bench] {wl.name}: generating and uploading")
    res = Resident(wl)
    ms = time_launches(res.softmax, res.n, steps, warmup)
    gbps = wl.bytes / (ms * 1e-3) / 1e9
    d = {"workload": wl.name, "rows": wl.rows, "cols": wl.cols, "dtype": wl.dtype,
         "kernel": kernel_name(res), "buffers": res.n, "us": round(ms * 1e3, 3),
         "gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4)}
    if oracle_timing:
        d["oracle_1core"] = oracle_rate(res.x_host, wl)
    if with_unfused:
        import torch
        nbytes = binding.unfused_workspace_bytes(wl.rows, wl.cols, res.code)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ums = time_launches(lambda i: binding.unfused_5op(res.ins[i].data_ptr(), res.outs[i].data_ptr(), wl.rows,
                                                           wl.cols, wl.cols, res.code, ws.data_ptr(), nbytes,
                                                           res.stream), res.n, steps, warmup)
        d["unfused_5op_us"] = round(ums * 1e3, 3)
        d["fused_speedup_over_unfused"] = round(ums / ms, 3)
        del ws
    if with_copy:
        cms = time_launches(res.copy, res.n, steps, warmup)
        d["copy_kernel_gbps"] = round(wl.bytes / (cms * 1e-3) / 1e9, 1)
        d["frac_of_copy"] = round(gbps / d["copy_kernel_gbps"], 4)
        if not light:
            mms = time_launches(res.memcpy, res.n, steps, warmup)
            d["memcpy_gbps"] = round(wl.bytes / (mms * 1e-3) / 1e9, 1)
    if light:
        log(f"[bench] {wl.name}: {d['us']} us  {d['gbps']} GB/s  ({100 * d['frac_of_peak']:.1f}% of 8 TB/s, "
            f"{d.get('frac_of_copy', 0):.3f} of copy)  kernel={d['kernel']}")
        d["_res"] = res
        return d
    # The same launches replayed from one captured graph: no host cost per launch.
    gms = time_graph(res, max(steps, res.n))
    d["graph_us"] = round(gms * 1e3, 3)
    d["graph_gbps"] = round(wl.bytes / (gms * 1e-3) / 1e9, 1)
    # Warm: one buffer pair launched over and over, so input and output stay in
    # the 256 MB Infinity Cache (and, for small shapes, in L2).  Not HBM-bound;
    # reported for reference only, never as the shape's number.
    wms = time_launches(lambda i: res.softmax(0), 1, steps, warmup)
    d["warm_us"] = round(wms * 1e3, 3)
    d["warm_gbps"] = round(wl.bytes / (wms * 1e-3) / 1e9, 1)
    log(f"[bench] {wl.name}: {d['us']} us  {d['gbps']} GB/s  ({100 * d['frac_of_peak']:.1f}% of 8 TB/s)"
        f"  kernel={d['kernel']}" + (f"  unfused 5-op {d['unfused_5op_us']} us ({d['fused_speedup_over_unfused']}x)"
                                     if "unfused_5op_us" in d else ""))
    d["_res"] = res
    return d


# The device code of the fused softmax kernels (attention and the unfused
# baseline are separate kernels and do not change the softmax's traffic).  The
# host side (softmax_abi.hip: validation, dispatch, launch) is left out; the
# kernel a stored counter run measured must instead be the one the dispatch
# picks now (stored_traffic).
SOFTMAX_SOURCES = ("kernel_table.hpp", "softmax_kernels.hpp", "table_bf16.hip", "table_entries.inc",
                   "table_f16.hip", "table_f32.hip")


def _code_only(text: str) -> str:
    """C++ source without comments or blank lines (comments cannot change a kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest() -> str:
    """Hash of the softmax kernel sources' code, to tell whether stored counters still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_wise_softmax_amd", "csrc")
    for name in SOFTMAX_SOURCES:
        h.update(name.encode())
        h.update(_code_only(open(os.path.join(csrc, name)).read()).encode())
    return h.hexdigest()[:16]


def kernel_signature(info) -> str:
    """The start of the demangled name rocprofv3 reports for a table entry (KernelInfo):
    template, element type, elements per access, then waves and accesses (row kernels) or
    lanes, accesses and groups (packed)."""
    elem = {0: "F32", 1: "F16", 2: "BF16"}[info.dtype]
    tmpl = {"packed": "softmax_packed", "row": "softmax_row", "row_pf": "softmax_row_pf",
            "online": "softmax_online"}[info.variant]
    if info.variant == "packed":
        args = f"{info.lanes}, {info.vecs_per_lane}, {info.groups}"
    else:
        args = f"{info.lanes // 64}, {info.vecs_per_lane}"
    return f"void rws::{tmpl}<rws::{elem}, {info.vec_elems}, {args}, {'true' if info.causal else 'false'}"


def stored_traffic(workload: str, kernel_info=None) -> dict | None:
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on this
    device code and (when kernel_info is given) on the kernel the dispatch picks now."""
    path = os.path.join(PROFILE_DIR, f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    if kernel_info is not None and not kv.get("kernel", "").startswith(kernel_signature(kernel_info)):
        return None
    try:
        return {"bytes": float(kv["hbm_bytes_per_dispatch"]), "source": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError):
        return None


def cpu_baseline(res: Resident, budget_s: float) -> dict:
    """The CPU oracle (single-threaded fp64 C) on the same input, repeated for about budget_s seconds."""
    from oracle import oracle
    wl = res.wl
    x = res.x_host
    times = []
    # pinned to one core of those this process may use (the calling thread
    # only), so the figure does not move with the scheduler's migrations
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        t_all = time.perf_counter()
        ref = None
        while True:
            t0 = time.perf_counter()
            ref = oracle.softmax(x, wl.dtype)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all >= budget_s:
                break
    finally:
        os.sched_setaffinity(0, allowed)
    mean = sum(times) / len(times)
    # The oracle's result also checks the benchmarked GPU output (recomputed
    # here: the copy-ceiling timings reuse the output buffers).
    import torch
    res.softmax(0)
    torch.cuda.synchronize()
    y = res.output(0)
    if wl.dtype == "f32":
        yd = y.astype(np.float64)
    elif wl.dtype == "f16":
        yd = y.view(np.float16).astype(np.float64)
    else:
        yd = (y.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    err = float(np.max(np.abs(yd - ref)))
    out = {"value": round(wl.bytes / mean / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"the whole {wl.name} input, {len(times)} run(s), {mean:.2f} s each, "
                     f"single-threaded fp64 C pinned to core {core}, same GB/s formula",
           "gpu_max_abs_err_vs_oracle": err}
    out["all_threads"] = oracle_threaded(x, wl, max(2.0, budget_s / 3))
    return out


def oracle_threaded(x: np.ndarray, wl, budget_s: float) -> dict:
    """The same oracle function over contiguous row ranges, one POSIX thread per
    range (oracle_softmax_mt), for a multi-core reference figure."""
    from oracle import oracle
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.softmax_mt(x, wl.dtype, threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all >= budget_s:
            break
    mean = sum(times) / len(times)
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(wl.bytes / mean / 1e9, 3), "unit": "GB/s", "cores": threads,
            "sample": f"the whole {wl.name} input split into {threads} row ranges, {len(times)} run(s), "
                      f"{mean:.3f} s each", "cpu": cpu}


ORACLE_SAMPLE_ELEMS = 1 << 21  # rows of about this many elements time the oracle on the large inputs


def oracle_rate(x: np.ndarray, wl) -> dict:
    """The single-threaded fp64 oracle on this shape's input, pinned to one core:
    the whole input when it has at most ORACLE_SAMPLE_ELEMS * 16 elements (best
    of 3 for inputs under 1 MB, one run otherwise), else the leading rows of
    about ORACLE_SAMPLE_ELEMS elements.  GB/s by the metric's formula on the
    rows timed."""
    from oracle import oracle
    rows = wl.rows if wl.rows * wl.cols <= ORACLE_SAMPLE_ELEMS * 16 else max(1, ORACLE_SAMPLE_ELEMS // wl.cols)
    part = np.ascontiguousarray(x[:rows])
    reps = 3 if part.nbytes < 1_000_000 else 1
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.softmax(part, wl.dtype)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
    finally:
        os.sched_setaffinity(0, allowed)
    nbytes = W.algorithmic_bytes(rows, wl.cols, wl.dtype)
    return {"rows_timed": rows, "seconds": round(best, 4), "gbps": round(nbytes / best / 1e9, 3),
            "runs": reps, "cores": 1}


def sweep(steps: int, warmup: int, keys: list | None = None) -> list:
    """Every fitting table kernel at every width of the sweep, bf16 and fp32
    (or at the workloads named in `keys`)."""
    table = binding.kernel_table()
    rows_out = []
    if keys is None:
        keys = [f"c5_{dt}_{w}" for dt in ("bf16", "f32") for w in W.SWEEP_WIDTHS]
    for key in keys:
        if True:
            wl = W.WORKLOADS[key]
            dt, w = wl.dtype, wl.cols
            res = Resident(wl)
            chosen = kernel_name(res)
            results = []
            spin_up(res.softmax, res.n, SPIN_S)  # once per width; the kernels then follow each other closely
            for k in table:
                if k.causal or "any_" in k.name:
                    continue  # the sweep times the plain softmax on the aligned kernels
                if not binding.kernel_fits(k.kid, res.ins[0].data_ptr(), res.outs[0].data_ptr(), wl.cols,
                                           wl.cols, res.code):
                    continue
                if k.max_cols > 0 and k.max_cols >= 4 * wl.cols:  # far too wide: wastes most lanes
                    continue
                ms = time_launches(lambda i, kid=k.kid: res.softmax(i, kid), res.n, steps, warmup, spin_s=0.02)
                results.append((wl.bytes / (ms * 1e-3) / 1e9, k.name, ms * 1e3))
            results.sort(reverse=True)
            best = results[0]
            chosen_gbps = next(g for g, n, _ in results if n == chosen) if any(n == chosen for _, n, _ in results) else None
            line = {"workload": wl.name, "key": key, "dtype": dt, "cols": w, "rows": wl.rows, "dispatch": chosen,
                    "dispatch_gbps": round(chosen_gbps, 1) if chosen_gbps else None,
                    "best": best[1], "best_gbps": round(best[0], 1),
                    "top5": [(n, round(g, 1)) for g, n, _ in results[:5]],
                    "all": [(n, round(g, 1)) for g, n, _ in results]}
            log(json.dumps(line))
            rows_out.append(line)
            del res
    # the narrow/wide crossover: widest width a packed kernel wins, narrowest a
    # one-workgroup-per-row kernel wins
    crossings = []
    for dt in ("bf16", "f32"):
        mine = [r for r in rows_out if r["dtype"] == dt and r["key"].startswith("c5_")]
        if not mine:
            continue
        packed = [r["cols"] for r in mine if r["best"].startswith("packed")]
        row = [r["cols"] for r in mine if r["best"].startswith(("row_", "rowpf_"))]
        cross = {"crossover": dt, "packed_wins_up_to_cols": max(packed) if packed else None,
                 "row_wins_from_cols": min(row) if row else None}
        log(json.dumps(cross))
        crossings.append(cross)
    return rows_out + crossings


# ------------------------------------------------------------ profile summaries

def summarize_sweep(sweep_json: str) -> None:
    """Write profiles/sweep_c5_widths.md (the crossover report) from `bench.py --sweep --sweep-out` JSON,
    or profiles/sweep_fixed_shapes.md when the sweep ran on other workloads (--sweep-keys)."""
    rows = json.load(open(sweep_json))
    src = os.path.relpath(os.path.abspath(sweep_json), ROOT)
    keys = [r["key"] for r in rows if "key" in r]
    c5 = all(k.startswith("c5_") for k in keys)
    vocab = all(k.startswith("vocab_") for k in keys)
    title = ("every plain table kernel at every c5 width" if c5 else
             "every plain table kernel at vocabulary-sized widths, 24576 to 151936 columns" if vocab else
             "every plain table kernel at the exact shapes " + ", ".join(keys))
    cmd = f"    python3 bench.py --sweep --sweep-out {src}" if c5 else \
        f"    python3 bench.py --sweep --sweep-keys {','.join(keys)} --sweep-out {src}"
    out = [f"# Kernel sweep on MI355X (gfx950): {title}", "",
           "Commands (repository root):", "",
           cmd,
           f"    python3 bench.py --summarize-sweep {src}", "",
           ("About 200 MB of input per tensor" if c5 or vocab else "The workloads' exact shapes") +
           ", rotating buffer sets of at least 1 GiB, 0.3 s spin-up per shape; GB/s by",
           "the metric's 2·rows·cols·size bytes.  `pick` is the kernel the width dispatch chooses, `best` the fastest",
           "kernel measured; the last column lists the next four.", "",
           "| dtype | cols | rows | pick | pick GB/s | best | best GB/s | next |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        if "cols" not in r:
            continue
        nxt = ", ".join(f"{n} {g:.0f}" for n, g in r["top5"][1:5])
        out.append(f"| {r['dtype']} | {r['cols']} | {r['rows']} | {r['dispatch']} | {r['dispatch_gbps']:.0f} | "
                   f"{r['best']} | {r['best_gbps']:.0f} | {nxt} |")
    out.append("")
    for r in rows:
        if "crossover" in r and c5:
            out.append(f"- {r['crossover']}: the packed kernel (several rows per wave) wins up to "
                       f"{r['packed_wins_up_to_cols']} columns; one workgroup per row wins from "
                       f"{r['row_wins_from_cols']} columns.")
    path = os.path.join(PROFILE_DIR, "sweep_c5_widths.md" if c5 else
                        "sweep_vocab_widths.md" if vocab else "sweep_fixed_shapes.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)


C3_BYTES = 8192 * 4096 * 2  # input bytes of the headline workload (8192 x 4096 fp16)


def softmax_dispatch_table(groups_csv: str) -> list:
    """Rows of the trace summary for the softmax kernels, one per (kernel, grid): a kernel
    template serves several shapes, so its overall average mixes them.  A row kernel's grid
    is one workgroup per row, which names the workload."""
    by_rows = collections.defaultdict(list)
    for key, wl in W.WORKLOADS.items():
        by_rows[(wl.rows, {"f32": "F32", "f16": "F16", "bf16": "BF16"}[wl.dtype])].append(key)
    rel = os.path.relpath(os.path.abspath(groups_csv), ROOT)
    out = ["", f"Softmax dispatches by launch grid, from the per-dispatch trace reduced with"
               f" `python3 bench.py --group-trace <trace csv> {rel}`; for a row kernel the grid is one workgroup"
               " per row, so its row count names the workload:", "",
           "| kernel | workgroups | threads each | workload | calls | average ns | min ns |", "|---|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(groups_csv)):
        name = r["Kernel_Name"]
        if "rws::softmax_" not in name:
            continue
        block = int(r["Workgroup_Size_X"])
        wgs = int(r["Grid_Size_X"]) // block
        tag = next((t for t in ("BF16", "F16", "F32") if f"rws::{t}," in name), "")
        label = ""
        if "softmax_row" in name:
            label = ", ".join(k for k in by_rows.get((wgs, tag), []) if not k.startswith("wide"))
        short = name.replace("void rws::", "").replace("(rws::Args)", "").replace("rws::", "")
        out.append(f"| `{short}` | {wgs} | {block} | {label} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                   f"{float(r['MinNs']):.0f} |")
    return out


def summarize_trace(stats_csv):
    """Write profiles/kernel_trace_bench.md from a rocprofv3 --stats kernel_stats.csv."""
    rows = list(csv.DictReader(open(stats_csv)))
    out_dir = os.path.relpath(os.path.dirname(os.path.abspath(stats_csv)), ROOT)
    out = ["# Kernel trace of the default benchmark run on MI355X (gfx950)", "",
           "Command (repository root):", "",
           f"    rocprofv3 --kernel-trace --stats --output-format csv -d {out_dir} -o bench -- python3 bench.py --no-cpu",
           *([f"    python3 bench.py --group-trace {out_dir}/bench_kernel_trace.csv "
              f"{os.path.relpath(os.path.abspath(stats_csv.replace('_kernel_stats.csv', '_dispatch_groups.csv')), ROOT)}"]
             if os.path.exists(stats_csv.replace("_kernel_stats.csv", "_dispatch_groups.csv")) else []),
           f"    python3 bench.py --summarize-trace {os.path.relpath(os.path.abspath(stats_csv), ROOT)}",
           "",
           "bench.py launches each kernel and shape untimed for 0.3 s (clock spin-up), then 50 warm-up + 200 timed"
           " launches, over rotating buffer sets of at least 1 GiB; the averages below cover all of them.",
           "Kernels, by template arguments `<element, elements per access, waves per row, accesses per lane, causal,"
           " line shift, any alignment>`:",
           "",
           "- `softmax_row_pf<F32,4,4,1,false,true,false>`: c1 128x1000 fp32 (4000-byte rows, line-shifted; few rows:"
           " the persistent twin);",
           "- `softmax_row_pf<F32,4,4,2,false,false,false>`: c2 2048x2048 fp32 (mask written in as -inf);",
           "- `softmax_row_pf<F32,4,4,2,true,false,false>`: c2 with the mask and 1/8 scale fused (raw scores in);",
           "- `softmax_row<F16,8,4,2,false,false,false>`: c3 8192x4096 fp16 (the headline);",
           "- `softmax_row<F32,4,8,2,false,false,false>`: c4 4096x4096 fp32;",
           "- `softmax_packed<...>` and `softmax_row<...>` at the 24 width-sweep tensors (c5), each once per width;",
           "- `copy16<4>` and `__amd_rocclr_copyBuffer`: the same-size copy references, for every shape; `copy16<4>`,"
           " `read16<4>` and `write16<4>` also at 8 MiB-1 GiB (the copy-ceiling table);",
           "- `unfused_reduce` / `unfused_elementwise`: the five-kernel unfused softmax on c3 and c4 (max, sub, exp, sum, div);",
           "- few, wide rows (8 x 1048576 fp32, 32 x 262144 bf16): `softmax_split_stats` + `softmax_split_merge` +"
           " `softmax_split_norm` with `Slot = true` (softmax_fwd's split, pairs kept in the output), the same two"
           " without the merge and `Slot = false` (softmax_fwd_split, caller workspace), and the width's"
           " one-workgroup-per-row kernel forced;",
           "- `attention_fwd_kernel<E,128,true>`: causal attention forward, batch 4, 32 heads, head dim 128"
           " (fp16 at 1024 and 4096 keys, bf16 at 4096; split by launch grid below).", "",
           "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    groups_csv = stats_csv.replace("_kernel_stats.csv", "_dispatch_groups.csv")
    if os.path.exists(groups_csv):
        out += softmax_dispatch_table(groups_csv)
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if not os.path.exists(trace_csv):  # the trace trimmed to the attention dispatches
        trace_csv = os.path.join(os.path.dirname(stats_csv), "attn_trace.csv")
    if not os.path.exists(trace_csv) and os.path.exists(groups_csv):
        trace_csv = groups_csv
    if os.path.exists(trace_csv):
        groups = {}  # (dtype, workgroups) -> [calls, total ns, min ns]
        for r in csv.DictReader(open(trace_csv)):
            if "attention_fwd_kernel" not in r["Kernel_Name"]:
                continue
            dt = "bf16" if "BF16" in r["Kernel_Name"] else "f16"
            key = (dt, int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
            if "AverageNs" in r:  # already reduced per (kernel, grid)
                n, tot, lo = int(r["Calls"]), float(r["AverageNs"]) * int(r["Calls"]), float(r["MinNs"])
            else:
                n, tot = 1, float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                lo = tot
            g = groups.setdefault(key, [0, 0.0, float("inf")])
            g[0], g[1], g[2] = g[0] + n, g[1] + tot, min(g[2], lo)
        if groups:
            out += ["", "Attention dispatches by launch grid (workgroups = 32 heads x 4 batch x queries / 128), from the"
                    " per-dispatch trace of the same run:", "",
                    "| dtype | workgroups | keys | calls | average ns | min ns |", "|---|---|---|---|---|---|"]
            for (dt, wg), (n, tot, lo) in sorted(groups.items()):
                heads, per_block = 4 * 32, 128  # batch x heads, queries per workgroup
                out.append(f"| {dt} | {wg} | {wg // heads * per_block} | {n} | {tot / n:.0f} | {lo:.0f} |")
    path = os.path.join(PROFILE_DIR, "kernel_trace_bench.md")
    open(path, "w").write("\n".join(out) + "\n")
    print(open(path).read())


def summarize_counters(fetch_csv, write_csv):
    """Write profiles/counters_c3_8192x4096_f16.txt from two rocprofv3 --pmc runs."""

    def avg(f, counter):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in d.items()}

    fe = avg(fetch_csv, "FETCH_SIZE")
    wr = avg(write_csv, "WRITE_SIZE")
    sm = next(k for k in fe if "softmax" in k)
    cp = next(k for k in fe if "copy16" in k)
    kib = C3_BYTES / 1024
    f_scale = kib / fe[cp]
    w_scale = kib / wr[cp]
    fetch_b = fe[sm] * f_scale * 1024
    write_b = wr[sm] * w_scale * 1024
    total = fetch_b + write_b
    alg = 2 * C3_BYTES
    rel = lambda f: os.path.relpath(os.path.abspath(f), ROOT)
    fdir, wdir = os.path.dirname(rel(fetch_csv)), os.path.dirname(rel(write_csv))
    txt = f"""# HBM traffic of the softmax kernel on 8192 x 4096 fp16 (c3_8192x4096_f16), MI355X (gfx950)
# Two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE), run from the repository root:
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fdir} -o c3 -- python3 bench.py --only c3 --no-cpu --steps 20 --warmup 5
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {wdir} -o c3 -- python3 bench.py --only c3 --no-cpu --steps 20 --warmup 5
# then: python3 bench.py --summarize-counters {rel(fetch_csv)} {rel(write_csv)}
# Counters are KiB per dispatch, averaged over each kernel's dispatches, and calibrated with
# the plain 16-byte copy kernel (softmax_bench_copy) of the same run, which reads and writes
# exactly {C3_BYTES} bytes: scale = known KiB / counter KiB.  FETCH_SIZE on this part
# reads about half of the bytes actually fetched (scale ~2.0); WRITE_SIZE reads true (~1.0).
kernel: {sm}
source_digest: {source_digest()}
copy_kernel_fetch_kib: {fe[cp]:.1f}
copy_kernel_write_kib: {wr[cp]:.1f}
fetch_scale: {f_scale:.5f}
write_scale: {w_scale:.5f}
softmax_fetch_kib_raw: {fe[sm]:.1f}
softmax_write_kib_raw: {wr[sm]:.1f}
softmax_fetch_bytes: {fetch_b:.0f}
softmax_write_bytes: {write_b:.0f}
hbm_bytes_per_dispatch: {total:.0f}
algorithmic_bytes_per_dispatch: {alg}
traffic_over_algorithmic: {total / alg:.5f}
"""
    path = os.path.join(PROFILE_DIR, "counters_c3_8192x4096_f16.txt")
    open(path, "w").write(txt)
    print(txt)


ATTN_COUNTER_PASSES = [
    "SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
]


def summarize_attention_counters(csvs):
    """Write profiles/counters_attention_b4_h32_d128_causal.txt from rocprofv3 --pmc CSVs of
    `bench.py --attention-only` (one CSV per counter pass)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))  # (kernel, grid) -> counter -> values
    for path in csvs:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "attention_fwd_kernel" in name:
                key = ("bf16" if "BF16" in name else "f16", int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            elif "copy16" in name:
                key = ("copy16", int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            else:
                continue
            per[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    mean = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in per.items()}
    copy_key = next((k for k in mean if k[0] == "copy16"), None)
    copy_bytes = 64 << 20
    lines = ["# Counters of the fused attention forward (causal, batch 4, 32 heads, head dim 128), MI355X (gfx950)",
             "# One rocprofv3 pass per line, run from the repository root:"]
    for i, ctr in enumerate(ATTN_COUNTER_PASSES):
        d = os.path.dirname(os.path.relpath(os.path.abspath(csvs[i]), ROOT)) if i < len(csvs) else "<dir>"
        lines.append(f"#   rocprofv3 --pmc {ctr} --output-format csv -d {d} -o a -- python3 bench.py --attention-only"
                     f" --steps 3 --warmup 1")
    lines += [f"# then: python3 bench.py --summarize-attention-counters "
              + " ".join(os.path.relpath(os.path.abspath(c), ROOT) for c in csvs),
              "# Values are per dispatch, averaged over each shape's dispatches.  FETCH_SIZE is scaled by what it",
              f"# reads for the plain copy kernel of the same run moving {copy_bytes} bytes each way; WRITE_SIZE likewise.",
              f"source_digest (attention.hip code): {attention_digest()}"]
    fscale = wscale = None
    if copy_key and "FETCH_SIZE" in mean[copy_key]:
        fscale = copy_bytes / 1024 / mean[copy_key]["FETCH_SIZE"]
    if copy_key and "WRITE_SIZE" in mean[copy_key]:
        wscale = copy_bytes / 1024 / mean[copy_key]["WRITE_SIZE"]
    for (dt, wgs), c in sorted(mean.items()):
        if dt == "copy16":
            continue
        n = wgs // 128 * 128  # 128 (batch, head) pairs, 128 queries per workgroup
        flops = 4.0 * 4 * 32 * 128 * n * (n + 1) / 2
        lines.append(f"\n[{dt} n={n} ({wgs} workgroups)]")
        for k in sorted(c):
            lines.append(f"{k}: {c[k]:.6g}")
        if "SQ_INSTS_MFMA" in c:
            lines.append(f"mfma_expected_from_flops: {flops / 32768:.6g}")
            lines.append(f"valu_per_mfma: {c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA'] - 1:.3f}  (SQ_INSTS_VALU counts the MFMAs too)")
        if "SQ_LDS_IDX_ACTIVE" in c and c["SQ_LDS_IDX_ACTIVE"] > 0:
            lines.append(f"lds_bank_conflict_fraction: {c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.4f}")
        if "TCC_HIT_sum" in c:
            lines.append(f"l2_hit_rate: {c['TCC_HIT_sum'] / (c['TCC_HIT_sum'] + c['TCC_MISS_sum']):.4f}")
        alg = 8.0 * 4 * 32 * n * 128  # Q, K, V read and O written once, 2 bytes each
        if "FETCH_SIZE" in c and fscale:
            lines.append(f"hbm_fetch_bytes: {c['FETCH_SIZE'] * 1024 * fscale:.6g}")
        if "WRITE_SIZE" in c and wscale:
            lines.append(f"hbm_write_bytes: {c['WRITE_SIZE'] * 1024 * wscale:.6g}")
        lines.append(f"algorithmic_bytes (q, k, v, o once): {alg:.6g}")
    txt = "\n".join(lines) + "\n"
    path = os.path.join(PROFILE_DIR, "counters_attention_b4_h32_d128_causal.txt")
    open(path, "w").write(txt)
    print(txt)


def attention_digest() -> str:
    """Hash of attention.hip's code (comments ignored)."""
    src = open(os.path.join(ROOT, "row_wise_softmax_amd", "csrc", "attention.hip")).read()
    return hashlib.sha256(_code_only(src).encode()).hexdigest()[:16]


def attention_only(steps: int, warmup: int) -> dict:
    """The attention shapes alone, plus one 64 MiB plain copy to calibrate the byte counters."""
    import torch
    n = (64 << 20) // 4
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        binding.bench_copy(a.data_ptr(), b.data_ptr(), n * 4, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del a, b
    return attention_shapes(steps, warmup)


COPY_SIZES_MIB = (8, 16, 32, 64, 128, 256, 512, 1024)


def copy_ceiling(steps: int, warmup: int, sizes=COPY_SIZES_MIB) -> list:
    """The copy kernel and its two directions alone (read-only, write-only) at each
    size in MiB of input, over rotating buffers of at least 1 GiB in all, timed like
    the softmax (spin-up, warm-up, events).  GB/s: bytes read plus bytes written."""
    import torch
    out = []
    stream = torch.cuda.current_stream().cuda_stream
    for mib in sizes:
        nbytes = mib << 20
        n = n_buffers(2 * nbytes)
        src = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
        dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
        r = {"mib": mib, "bytes": nbytes, "buffers": n}
        for mode, name in ((0, "copy"), (1, "read"), (2, "write")):
            ms = time_launches(lambda i, m=mode: binding.bench_stream(src[i].data_ptr(), dst[i].data_ptr(), nbytes, m,
                                                                       stream), n, steps, warmup)
            moved = 2 * nbytes if mode == 0 else nbytes
            r[f"{name}_us"] = round(ms * 1e3, 3)
            r[f"{name}_gbps"] = round(moved / (ms * 1e-3) / 1e9, 1)
        log(f"[bench] copy ceiling {mib} MiB: copy {r['copy_gbps']}  read {r['read_gbps']}  write {r['write_gbps']} GB/s")
        out.append(r)
        del src, dst
        torch.cuda.synchronize()
    return out


def trace_by_stream_size(trace_csv: str) -> dict:
    """Average dispatch ns of copy16 / read16 / write16 per input size in MiB, from a
    rocprofv3 kernel-trace CSV (the grid is size / 16 KiB workgroups of 256 threads)."""
    got = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        kind = next((k for k in ("copy16", "read16", "write16") if f"rws::{k}<" in name), None)
        if kind is None:
            continue
        mib = int(r["Grid_Size_X"]) // 256 * 16384 // (1 << 20)
        if "AverageNs" in r:  # a per-(kernel, grid) summary of the trace: weight by its calls
            got[(kind, mib)] += [float(r["AverageNs"])] * int(r["Calls"])
        else:
            got[(kind, mib)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: sum(v) / len(v) for k, v in got.items()}


CHUNK_COPY_MIB = 192  # about the c5 tensors' 200 MB; a multiple of every chunk shape


def chunk_copy(steps: int, warmup: int, mib: int = CHUNK_COPY_MIB, rounds: int = 3) -> list:
    """The row kernels' access pattern without their arithmetic: softmax_bench_chunk_copy
    at every shape, and the plain copy kernel, on `mib` MiB over rotating buffers; the
    median of `rounds` interleaved timings each."""
    import torch
    nbytes = mib << 20
    n = n_buffers(2 * nbytes)
    src = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    stream = torch.cuda.current_stream().cuda_stream
    cands = {"copy16": lambda i: binding.bench_copy(src[i].data_ptr(), dst[i].data_ptr(), nbytes, stream)}
    for w, v in binding.CHUNK_COPY_SHAPES:
        cands[f"w{w}_v{v}"] = (lambda i, w=w, v=v: binding.bench_chunk_copy(src[i].data_ptr(), dst[i].data_ptr(),
                                                                            nbytes, w, v, stream))
    got = {k: [] for k in cands}
    spin_up(cands["copy16"], n, SPIN_S)
    for _ in range(rounds):
        for k, f in cands.items():
            ms = time_launches(f, n, steps, warmup, spin_s=0.02)
            got[k].append(2 * nbytes / (ms * 1e-3) / 1e9)
    out = []
    for k, vals in got.items():
        w, v = (None, None) if k == "copy16" else (int(k.split("_")[0][1:]), int(k.split("_")[1][1:]))
        out.append({"kernel": k, "waves": w, "accesses": v, "chunk_kib": (w * 64 * v * 16 // 1024) if w else None,
                    "gbps": round(float(np.median(vals)), 1), "runs": [round(x, 1) for x in vals]})
        log(f"[bench] chunk copy {k}: {out[-1]['gbps']} GB/s")
    del src, dst
    torch.cuda.synchronize()
    return out


SPLIT_CROSS_ROWS = (8, 16, 32, 64, 128, 192, 256)
SPLIT_CROSS_ROW_KIB = (64, 128, 192, 224, 256, 384, 512, 1024, 2048, 4096)
SPLIT_CROSS_MAX_BYTES = 512 << 20


def split_crossover(steps: int, warmup: int) -> list:
    """Few, very wide rows: for each dtype, row size and row count, the width's
    one-workgroup-per-row kernel (softmax_fwd_variant at softmax_select_variant's
    pick), softmax_fwd_split with a workspace (always split), and softmax_fwd
    itself (which splits through its output where its rule says so).  Seeded
    N(0, 1) inputs drawn on the device, rotating buffers of at least 768 MiB."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for dt in ("f32", "f16", "bf16"):
        code, esz, tdt = W.dtype_code(dt), (4 if dt == "f32" else 2), torch_dtype(dt)
        for kib in SPLIT_CROSS_ROW_KIB:
            cols = (kib << 10) // esz
            variant, block = binding.softmax_select_variant(cols, code)
            for rows in SPLIT_CROSS_ROWS:
                nbytes = rows * cols * esz
                if nbytes > SPLIT_CROSS_MAX_BYTES:
                    continue
                n = max(1, -(-(768 << 20) // (2 * nbytes)))
                g = torch.Generator(device="cuda").manual_seed(rows * 131 + kib)
                xs = [torch.randn((rows, cols), generator=g, device="cuda").to(tdt) for _ in range(n)]
                ys = [torch.empty_like(x) for x in xs]
                wsb = binding.split_workspace_bytes(rows, cols, code)
                ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
                kid = binding.softmax_select(xs[0].data_ptr(), ys[0].data_ptr(), cols, cols, code, rows=rows)
                runs = {
                    "one_wg_per_row": lambda i: binding.softmax_fwd_variant(xs[i].data_ptr(), ys[i].data_ptr(), rows,
                                                                            cols, cols, code, variant, block, stream),
                    "split_workspace": lambda i: binding.softmax_fwd_split(xs[i].data_ptr(), ys[i].data_ptr(), rows,
                                                                           cols, cols, code, ws.data_ptr(), wsb, 1,
                                                                           stream),
                    "softmax_fwd": lambda i: binding.softmax_fwd(xs[i].data_ptr(), ys[i].data_ptr(), rows, cols, cols,
                                                                 code, stream)}
                us = {k: round(time_launches(f, n, steps, warmup, spin_s=0.02) * 1e3, 2) for k, f in runs.items()}
                r = {"dtype": dt, "row_kib": kib, "rows": rows, "cols": cols,
                     "softmax_fwd_path": "split via out" if kid == binding.SPLIT_KERNEL else "table", **us}
                log(f"[bench] split crossover {dt} {kib} KiB x {rows}: {us}  ({r['softmax_fwd_path']})")
                out.append(r)
                del xs, ys, ws
                torch.cuda.empty_cache()
    return out


def summarize_split_crossover(json_path: str) -> None:
    """Write profiles/split_crossover.md from `bench.py --split-crossover --split-out` JSON."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    out = ["# Few, very wide rows: one workgroup per row against the split path, MI355X (gfx950)", "",
           "Commands (repository root):", "",
           f"    python3 bench.py --split-crossover --split-out {src}",
           f"    python3 bench.py --summarize-split-crossover {src}", "",
           "Microseconds per call over rotating buffers of at least 768 MiB, seeded N(0, 1) inputs.  `one wg/row`:",
           "the width's one-workgroup-per-row kernel forced (softmax_fwd_variant at softmax_select_variant's pick);",
           "`split+ws`: softmax_fwd_split with a caller workspace, always split (two kernels); `softmax_fwd`: the",
           "library's own choice, which splits through its output where the path column says so (two kernels up to",
           "1024 tiles in all, else three).",
           "`gain` = one wg/row / softmax_fwd.", "",
           "| dtype | row KiB | rows | one wg/row us | split+ws us | softmax_fwd us | softmax_fwd path | gain |",
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['dtype']} | {r['row_kib']} | {r['rows']} | {r['one_wg_per_row']:.1f} | "
                   f"{r['split_workspace']:.1f} | {r['softmax_fwd']:.1f} | {r['softmax_fwd_path']} | "
                   f"{r['one_wg_per_row'] / r['softmax_fwd']:.2f} |")
    path = os.path.join(PROFILE_DIR, "split_crossover.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


RAGGED_WIDTHS = {"f32": (600, 900, 960, 1000, 1020), "bf16": (1200, 1800, 2000, 2040)}
RAGGED_ROWS = (2048, 4096, 8192, 16384, 65536)
RAGGED_SHAPES = ("row_{}_w4_v1", "rowpf_{}_w4_v1", "row_{}_w2_v2", "rowpf_{}_w2_v2", "row_{}_w4_v2")


def ragged_rows(steps: int, warmup: int) -> list:
    """Ragged widths of 129..255 16-byte accesses (aligned, contiguous) at
    2 K-64 K rows: softmax_fwd and each candidate row shape forced (four waves
    of one access, two of two, four of two; plain and persistent).  Seeded
    N(0, 1) inputs drawn on the device, rotating buffers of at least 1 GiB,
    the best of three interleaved timings each."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    table = binding.kernel_table()
    ids = {k.name: k.kid for k in table}
    out = []
    for dt, widths in RAGGED_WIDTHS.items():
        code, esz, tdt = W.dtype_code(dt), (4 if dt == "f32" else 2), torch_dtype(dt)
        for cols in widths:
            for rows in RAGGED_ROWS:
                nbytes = rows * cols * esz
                n = n_buffers(2 * nbytes)
                g = torch.Generator(device="cuda").manual_seed(cols * 7 + rows)
                xs = [torch.randn((rows, cols), generator=g, device="cuda").to(tdt) for _ in range(n)]
                ys = [torch.empty_like(x) for x in xs]
                kid = binding.softmax_select(xs[0].data_ptr(), ys[0].data_ptr(), cols, cols, code, rows=rows)
                runs = {"softmax_fwd": lambda i: binding.softmax_fwd(xs[i].data_ptr(), ys[i].data_ptr(), rows, cols,
                                                                     cols, code, stream)}
                for shape in RAGGED_SHAPES:
                    k = ids[shape.format(dt)]
                    runs[shape.format(dt)] = (lambda k: lambda i: binding.softmax_fwd_kernel(
                        k, xs[i].data_ptr(), ys[i].data_ptr(), rows, cols, cols, code, stream))(k)
                best = {k: 0.0 for k in runs}
                for _ in range(3):
                    for k, f in runs.items():
                        ms = time_launches(f, n, steps, warmup, spin_s=0.02)
                        best[k] = max(best[k], 2 * nbytes / (ms * 1e-3) / 1e9)
                r = {"dtype": dt, "rows": rows, "cols": cols, "accesses": cols * esz // 16,
                     "kernel": table[kid].name, **{k: round(v, 1) for k, v in best.items()}}
                log(f"[bench] ragged {dt} {rows}x{cols}: {r}")
                out.append(r)
                del xs, ys
                torch.cuda.empty_cache()
    return out


def summarize_ragged_rows(json_path: str) -> None:
    """Write profiles/ragged_widths_rows.md from `bench.py --ragged-rows --ragged-out` JSON."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    heads = [s.format("dt").replace("_dt_", " ").replace("_", "") for s in RAGGED_SHAPES]
    out = ["# Ragged widths (129..255 16-byte accesses) across row counts, MI355X (gfx950)", "",
           "Commands (repository root):", "",
           f"    python3 bench.py --ragged-rows --ragged-out {src}",
           f"    python3 bench.py --summarize-ragged-rows {src}", "",
           "Contiguous tensors of widths a multiple of 16 bytes, seeded N(0, 1) inputs, rotating buffers of at",
           "least 1 GiB, best of three interleaved timings; GB/s by the metric's 2·rows·cols·size bytes.  The",
           "shape columns force one kernel (`w4v1`: four waves of one 16-byte access per lane, `w2v2`: two",
           "waves of two, `w4v2`: four waves of two; `rowpf`: the persistent twin).  `pick / best`: softmax_fwd",
           "against the fastest column of its line.", "",
           "| dtype | cols | accesses | rows | pick | softmax_fwd | " + " | ".join(heads) + " | pick / best |",
           "|---|---|---|---|---|---|" + "---|" * len(heads) + "---|"]
    for r in rows:
        vals = [r[s.format(r["dtype"])] for s in RAGGED_SHAPES]
        best = max(vals + [r["softmax_fwd"]])
        out.append(f"| {r['dtype']} | {r['cols']} | {r['accesses']} | {r['rows']} | {r['kernel']} | "
                   f"{r['softmax_fwd']:.0f} | " + " | ".join(f"{v:.0f}" for v in vals) +
                   f" | {r['softmax_fwd'] / best:.3f} |")
    path = os.path.join(PROFILE_DIR, "ragged_widths_rows.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


PAST_POW2_CHUNKS = (300, 340, 375, 420, 520, 580, 625, 700, 750, 800, 960, 1100, 1250, 1400, 1500, 1650, 1950,
                    2200, 2500, 2800, 3300, 3800)
PAST_POW2_BYTES = (200_000_000, 50_000_000)
# fp32 rows that fill the two-access shape exactly, across row counts
FULL_ROWS_POINTS = tuple(("f32", nacc, rows) for nacc in (256, 512) for rows in (8192, 12288, 16384, 24576, 49152))
# jobs just past the persistent twin's two rounds (16 waves: 1024 rows; 8 waves: 2048)
ROUND_POINTS = tuple([("bf16", 2048, r) for r in (1025, 1100, 1200, 1280, 1400, 1700)] +
                     [("bf16", 1600, r) for r in (1025, 1200, 1280, 1400)] +
                     [("f32", 2048, r) for r in (1025, 1200, 1400, 1700)] +
                     [("bf16", 1024, r) for r in (2049, 2200, 2560, 2800)] +
                     [("f32", 1024, r) for r in (2049, 2400)])


def past_pow2(steps: int, warmup: int) -> list:
    """Aligned rows of 300..3800 16-byte accesses (chunk counts between powers
    of two), bf16 and fp32, at about 200 MB and 50 MB per tensor, and fp32 rows
    of exactly 256 and 512 accesses at 8 K-48 K rows, and jobs of 1 K-3 K
    rows just past the persistent twin's two rounds: softmax_fwd and every row
    kernel (widened or, 16-bit, stored values; persistent too where the job has
    at most 4096 rows) whose slots hold the row at most twice over.  Seeded N(0, 1) inputs drawn on the
    device, rotating buffers of at least 1 GiB, the median of three interleaved
    timings each."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    table = binding.kernel_table()
    out = []
    points = [(dt, nacc, size // (nacc * 16)) for dt in ("bf16", "f32") for nacc in PAST_POW2_CHUNKS
              for size in PAST_POW2_BYTES] + list(FULL_ROWS_POINTS) + list(ROUND_POINTS)
    for dt, nacc, rows in points:
        code, esz, tdt = W.dtype_code(dt), (4 if dt == "f32" else 2), torch_dtype(dt)
        cols = nacc * 16 // esz
        nbytes = rows * cols * esz
        n = n_buffers(2 * nbytes)
        g = torch.Generator(device="cuda").manual_seed(cols + rows)
        xs = [torch.randn((rows, cols), generator=g, device="cuda").to(tdt) for _ in range(n)]
        ys = [torch.empty_like(x) for x in xs]
        kid = binding.softmax_select(xs[0].data_ptr(), ys[0].data_ptr(), cols, cols, code, rows=rows)
        runs = {"softmax_fwd": lambda i: binding.softmax_fwd(xs[i].data_ptr(), ys[i].data_ptr(), rows, cols,
                                                             cols, code, stream)}
        for k in table:
            if k.dtype != code or k.causal or not k.name.startswith(("row_", "row16_", "rowpf_")):
                continue
            if k.name.startswith("rowpf_") and rows > 4096:
                continue  # the persistent twins matter for jobs of few rows only
            if nacc <= k.lanes * k.vecs_per_lane <= 2 * nacc:
                runs[k.name] = (lambda kk: lambda i: binding.softmax_fwd_kernel(
                    kk, xs[i].data_ptr(), ys[i].data_ptr(), rows, cols, cols, code, stream))(k.kid)
        spin_up(runs["softmax_fwd"], n, 0.2)
        got = {k: [] for k in runs}
        for _ in range(3):
            for k, f in runs.items():
                ms = time_launches(f, n, steps, warmup, spin_s=0.01)
                got[k].append(2 * nbytes / (ms * 1e-3) / 1e9)
        r = {"dtype": dt, "rows": rows, "cols": cols, "accesses": nacc, "kernel": table[kid].name,
             "gbps": {k: round(sorted(v)[1], 1) for k, v in got.items()}}
        log(f"[bench] past-pow2 {dt} {rows}x{cols}: {r}")
        out.append(r)
        del xs, ys
        torch.cuda.empty_cache()
    return out


def summarize_past_pow2(json_path: str) -> None:
    """Write profiles/past_pow2_widths.md from `bench.py --past-pow2 --past-pow2-out` JSON."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    out = ["# Rows between powers of two of 16-byte accesses: row shapes by waves and accesses per lane, MI355X (gfx950)",
           "", "Commands (repository root):", "",
           f"    python3 bench.py --past-pow2 --past-pow2-out {src}",
           f"    python3 bench.py --summarize-past-pow2 {src}", "",
           "Contiguous aligned tensors of about 200 MB and 50 MB, seeded N(0, 1) inputs, rotating buffers of at",
           "least 1 GiB, median of three interleaved timings; GB/s by the metric's 2·rows·cols·size bytes.",
           "`wWvV`: the plain row kernel forced on W waves of V accesses per lane (`16wWvV`: the 16-bit kernel",
           "that keeps stored values, `pfwWvV`: the persistent twin, timed on jobs of at most 4096 rows), the",
           "shapes whose slots hold the row at most twice over.  `pick / best`: softmax_fwd against the fastest shape of its line.", "",
           "| dtype | cols | accesses | rows | pick | softmax_fwd | best shape | best | next | pick / best |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        g = r["gbps"]
        shapes = sorted(((v, k) for k, v in g.items() if k != "softmax_fwd"), reverse=True)
        best = max([g["softmax_fwd"]] + [v for v, _ in shapes])
        short = lambda k: ({"row16": "16", "rowpf": "pf"}.get(k.split("_")[0], "") +
                           k.split("_", 2)[2].replace("_", ""))
        nxt = ", ".join(f"{short(k)} {v:.0f}" for v, k in shapes[1:4])
        bname = short(shapes[0][1])
        out.append(f"| {r['dtype']} | {r['cols']} | {r['accesses']} | {r['rows']} | {r['kernel']} | "
                   f"{g['softmax_fwd']:.0f} | {bname} | {shapes[0][0]:.0f} | {nxt} | {g['softmax_fwd'] / best:.3f} |")
    path = os.path.join(PROFILE_DIR, "past_pow2_widths.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


FEW_ROWS_WIDTHS = {"f32": (1024, 2048, 4096, 8192), "bf16": (2048, 4096, 8192, 16384)}
FEW_ROWS = (256, 512, 1024, 2048, 4096)


def few_rows(steps: int, warmup: int) -> list:
    """Jobs of few rows (256-4096) at aligned widths of 4-32 KiB: softmax_fwd
    and every persistent row shape (the twin family) whose slots hold the row
    at most twice over, each forced.  Seeded N(0, 1) inputs drawn on the device,
    rotating buffers of at least 1 GiB, the best of three interleaved timings."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    table = binding.kernel_table()
    out = []
    for dt, widths in FEW_ROWS_WIDTHS.items():
        code, esz, tdt = W.dtype_code(dt), (4 if dt == "f32" else 2), torch_dtype(dt)
        for cols in widths:
            for rows in FEW_ROWS:
                nbytes = rows * cols * esz
                n = n_buffers(2 * nbytes)
                g = torch.Generator(device="cuda").manual_seed(cols * 11 + rows)
                xs = [torch.randn((rows, cols), generator=g, device="cuda").to(tdt) for _ in range(n)]
                ys = [torch.empty_like(x) for x in xs]
                x0, y0 = xs[0].data_ptr(), ys[0].data_ptr()
                kid = binding.softmax_select(x0, y0, cols, cols, code, rows=rows)
                runs = {"softmax_fwd": lambda i: binding.softmax_fwd(xs[i].data_ptr(), ys[i].data_ptr(), rows, cols,
                                                                     cols, code, stream)}
                for k in table:
                    if (k.dtype == code and k.variant == "row_pf" and not k.causal and not k.name.startswith("any_")
                            and k.max_cols <= 2 * cols and binding.kernel_fits(k.kid, x0, y0, cols, cols, code)):
                        runs[k.name] = (lambda kk: lambda i: binding.softmax_fwd_kernel(
                            kk, xs[i].data_ptr(), ys[i].data_ptr(), rows, cols, cols, code, stream))(k.kid)
                best = {k: 0.0 for k in runs}
                for _ in range(3):
                    for k, f in runs.items():
                        ms = time_launches(f, n, steps, warmup, spin_s=0.02)
                        best[k] = max(best[k], 2 * nbytes / (ms * 1e-3) / 1e9)
                r = {"dtype": dt, "rows": rows, "cols": cols, "kernel": table[kid].name,
                     "gbps": {k: round(v, 1) for k, v in best.items()}}
                log(f"[bench] few rows {dt} {rows}x{cols}: {r}")
                out.append(r)
                del xs, ys
                torch.cuda.empty_cache()
    return out


def summarize_few_rows(json_path: str) -> None:
    """Write profiles/few_rows_shapes.md from `bench.py --few-rows --few-out` JSON."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    out = ["# Few rows: the persistent row shapes at 256-4096 rows, MI355X (gfx950)", "",
           "Commands (repository root):", "",
           f"    python3 bench.py --few-rows --few-out {src}",
           f"    python3 bench.py --summarize-few-rows {src}", "",
           "Contiguous tensors, seeded N(0, 1) inputs, rotating buffers of at least 1 GiB, best of three interleaved",
           "timings; GB/s by the metric's 2·rows·cols·size bytes.  Each persistent row shape (`rowpf_<dtype>_w<W>_v<V>`:",
           "W waves per row, V 16-byte accesses per lane, grid = resident workgroups) whose slots hold the row at most",
           "twice over is forced; `pick / best` is softmax_fwd against the fastest of them (or itself).", "",
           "| dtype | cols | rows | pick | softmax_fwd GB/s | best shape | best GB/s | pick / best | next three |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        g = dict(r["gbps"])
        pick = g.pop("softmax_fwd")
        ranked = sorted(g.items(), key=lambda kv: -kv[1])
        bname, bval = ranked[0] if ranked else ("-", 0.0)
        top = max(bval, pick)
        nxt = ", ".join(f"{k.split('_', 2)[2]} {v:.0f}" for k, v in ranked[1:4])
        out.append(f"| {r['dtype']} | {r['cols']} | {r['rows']} | {r['kernel']} | {pick:.0f} | {bname} | {bval:.0f} | "
                   f"{pick / top:.3f} | {nxt} |")
    path = os.path.join(PROFILE_DIR, "few_rows_shapes.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


ODD_WIDTHS = {"f32": (1001, 1025, 2049, 3001, 4097, 8193, 16385, 32001, 50257),
              "bf16": (1001, 2049, 4097, 8193, 16385, 32001, 50257)}


def odd_widths(steps: int, warmup: int) -> list:
    """Widths that are not a multiple of 16 bytes, at about 200 MB per tensor:
    softmax_fwd (the any-alignment kernels), the scalar path forced (what such
    widths ran on before), and the aligned width just below (the same row count,
    on the aligned kernels).  Seeded N(0, 1) inputs drawn on the device,
    rotating buffers of at least 1 GiB, the best of three timings each."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    table = binding.kernel_table()
    out = []
    for dt, widths in ODD_WIDTHS.items():
        code, esz, tdt = W.dtype_code(dt), (4 if dt == "f32" else 2), torch_dtype(dt)
        vec = 16 // esz
        for cols in widths:
            rows = max(64, int(200e6 // (cols * esz)))
            nbytes = rows * cols * esz
            n = n_buffers(2 * nbytes)
            g = torch.Generator(device="cuda").manual_seed(cols)
            xs = [torch.randn((rows, cols), generator=g, device="cuda").to(tdt) for _ in range(n)]
            ys = [torch.empty_like(x) for x in xs]
            kid = binding.softmax_select(xs[0].data_ptr(), ys[0].data_ptr(), cols, cols, code, rows=rows)
            # the scalar kernel softmax_fwd runs for input and output at different offsets in their chunks
            block = 64 * (1 if cols <= 512 else 4 if cols <= 8192 else 16)
            scalar = next(k.kid for k in table if k.dtype == code and k.variant == "online" and k.vec_elems == 1
                          and not k.causal and k.block == block)
            al = cols // vec * vec  # the aligned width below, as a view of the same buffers (pitch = cols)
            runs = {"softmax_fwd": lambda i: binding.softmax_fwd(xs[i].data_ptr(), ys[i].data_ptr(), rows, cols, cols,
                                                                 code, stream),
                    "scalar": lambda i: binding.softmax_fwd_kernel(scalar, xs[i].data_ptr(), ys[i].data_ptr(), rows,
                                                                   cols, cols, code, stream)}
            xa = [torch.randn((rows, al), generator=g, device="cuda").to(tdt) for _ in range(n)]
            ya = [torch.empty_like(x) for x in xa]
            runs["aligned_below"] = lambda i: binding.softmax_fwd(xa[i].data_ptr(), ya[i].data_ptr(), rows, al, al,
                                                                  code, stream)
            best = {k: 0.0 for k in runs}
            for _ in range(3):
                for k, f in runs.items():
                    ms = time_launches(f, n, steps, warmup, spin_s=0.05)
                    b = (nbytes if k != "aligned_below" else rows * al * esz) * 2
                    best[k] = max(best[k], b / (ms * 1e-3) / 1e9)
            r = {"dtype": dt, "rows": rows, "cols": cols, "aligned_cols": al,
                 "kernel": table[kid].name if kid >= 0 else "split", **{k: round(v, 1) for k, v in best.items()}}
            log(f"[bench] odd width {dt} {rows}x{cols}: {r}")
            out.append(r)
            del xs, ys, xa, ya
            torch.cuda.empty_cache()
    return out


def summarize_odd_widths(json_path: str) -> None:
    """Write profiles/odd_widths.md from `bench.py --odd-widths --odd-out` JSON."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    out = ["# Widths that are not a multiple of 16 bytes, MI355X (gfx950)", "",
           "Commands (repository root):", "",
           f"    python3 bench.py --odd-widths --odd-out {src}",
           f"    python3 bench.py --summarize-odd-widths {src}", "",
           "About 200 MB per tensor, contiguous (so consecutive rows start at every offset within a 16-byte chunk),",
           "seeded N(0, 1) inputs, rotating buffers of at least 1 GiB, best of three timings; GB/s by the metric's",
           "2·rows·cols·size bytes.  `softmax_fwd`: the library's pick (the any-alignment kernels); `scalar`: the",
           "element-by-element online kernel, forced -- what softmax_fwd runs when input and output sit at",
           "different offsets in their 16-byte chunks, and what every such width ran on before the any-alignment",
           "kernels; `aligned below`: softmax_fwd on the same row count at the largest 16-byte-multiple width below.",
           "",
           "| dtype | rows | cols | pick | softmax_fwd GB/s | scalar GB/s | gain | aligned below (cols) GB/s | / aligned |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['dtype']} | {r['rows']} | {r['cols']} | {r['kernel']} | {r['softmax_fwd']:.0f} | "
                   f"{r['scalar']:.0f} | {r['softmax_fwd'] / r['scalar']:.2f}x | {r['aligned_below']:.0f} "
                   f"({r['aligned_cols']}) | {r['softmax_fwd'] / r['aligned_below']:.3f} |")
    path = os.path.join(PROFILE_DIR, "odd_widths.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_chunk_copy(json_path: str, bench_json: str | None = None) -> None:
    """Write profiles/chunk_copy_shapes.md from `bench.py --chunk-copy --chunk-out` JSON and,
    optionally, a default bench line whose c5 shapes give each row kernel's own rate."""
    rows = json.load(open(json_path))
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    users = collections.defaultdict(list)
    if bench_json:
        line = json.loads(open(bench_json).read().strip().splitlines()[-1])
        for key, sh in line.get("shapes", {}).items():
            k = sh.get("kernel", "")
            if key.startswith("c5_") and k.startswith("row_"):
                _, dt, w, v = k.split("_")
                users[(int(w[1:]), int(v[1:]))].append(f"{dt} {sh['cols']}: {sh['gbps']:.0f}")
    cmd = [f"    python3 bench.py --chunk-copy --chunk-out {src}"]
    if bench_json:
        cmd.append(f"    python3 bench.py > {os.path.relpath(os.path.abspath(bench_json), ROOT)}")
    cmd.append(f"    python3 bench.py --summarize-chunk-copy {src}" +
               (f" {os.path.relpath(os.path.abspath(bench_json), ROOT)}" if bench_json else ""))
    out = ["# The row kernels' access pattern alone: copies in per-workgroup chunks, MI355X (gfx950)", "",
           "Commands (repository root):", "", *cmd, "",
           f"`softmax_bench_chunk_copy` on {CHUNK_COPY_MIB} MiB (about a c5 tensor): each workgroup of W waves copies one",
           "contiguous chunk of W x 64 x V 16-byte accesses the way the row kernels read and write a row (wave w its run of",
           "64 V accesses, all loads, a barrier, all stores), with no arithmetic.  `copy16` is the grid-stride copy kernel.",
           "Median of three interleaved timings over rotating buffers of at least 1 GiB; GB/s = 2 x size / time.  The",
           "last column lists the c5 widths whose dispatch pick is the row kernel of that shape, with that kernel's GB/s",
           "from the default bench run.", "",
           "| kernel | waves | accesses per lane | chunk KiB | GB/s | runs | softmax row kernels of this shape (GB/s) |",
           "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: (r["chunk_kib"] or 0, r["waves"] or 0)):
        use = "; ".join(users.get((r["waves"], r["accesses"]), []))
        out.append(f"| {r['kernel']} | {r['waves'] or ''} | {r['accesses'] or ''} | {r['chunk_kib'] or ''} | "
                   f"{r['gbps']:.0f} | {', '.join(f'{x:.0f}' for x in r['runs'])} | {use} |")
    path = os.path.join(PROFILE_DIR, "chunk_copy_shapes.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def group_trace(trace_csv: str, out_csv: str) -> None:
    """Reduce a rocprofv3 per-dispatch kernel trace to one line per (kernel, grid, workgroup):
    calls, average and minimum duration.  The full trace of a default run is too large to keep."""
    g = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        g[(r["Kernel_Name"][:160], r["Grid_Size_X"], r["Workgroup_Size_X"])].append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    with open(out_csv, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Calls", "AverageNs", "MinNs"])
        for (k, gx, wx), v in sorted(g.items()):
            w.writerow([k, gx, wx, len(v), sum(v) / len(v), min(v)])


def summarize_copy_sizes(json_path: str, trace_csv: str | None = None) -> None:
    """Write profiles/copy_ceiling_sizes.md from `bench.py --copy-sizes --copy-out` JSON
    (or from a default bench line, which carries the same table as copy_ceiling), with
    the per-dispatch averages of a rocprofv3 kernel trace of the same run if given."""
    d = json.load(open(json_path))
    rows = d["copy_ceiling"] if isinstance(d, dict) else d
    src = os.path.relpath(os.path.abspath(json_path), ROOT)
    trace = trace_by_stream_size(trace_csv) if trace_csv else {}
    # the event-timed table: a default bench line (its copy_ceiling) or a --copy-sizes file
    cmd = [f"    python3 bench.py > {src}" if isinstance(d, dict) else f"    python3 bench.py --copy-sizes --copy-out {src}"]
    if trace_csv:
        tdir = os.path.dirname(os.path.relpath(os.path.abspath(trace_csv), ROOT))
        if os.path.basename(trace_csv).startswith("bench_"):  # the default run's trace (bench.py --no-cpu)
            cmd.append(f"    rocprofv3 --kernel-trace --stats --output-format csv -d {tdir} -o bench -- "
                       f"python3 bench.py --no-cpu")
            cmd.append(f"    python3 bench.py --group-trace {tdir}/bench_kernel_trace.csv "
                       f"{os.path.relpath(os.path.abspath(trace_csv), ROOT)}")
        else:
            cmd.append(f"    rocprofv3 --kernel-trace --stats --output-format csv -d {tdir} -o cs -- "
                       f"python3 bench.py --copy-sizes --copy-out {tdir}/copy_sizes.json")
    cmd.append(f"    python3 bench.py --summarize-copy-sizes {src}" +
               (f" {os.path.relpath(os.path.abspath(trace_csv), ROOT)}" if trace_csv else ""))
    out = ["# Copy ceiling by size on MI355X (gfx950): the 16-byte copy kernel and its two directions", "",
           "Command (repository root):", "", *cmd, "",
           "Kernels: `softmax_bench_stream` modes 0 (copy, `copy16<4>`), 1 (read-only, `read16<4>`) and 2 (write-only,",
           "`write16<4>`), 256 threads, four 16-byte non-temporal accesses per thread in flight, grid-stride.  Rotating",
           "buffer sets of at least 1 GiB, 0.3 s spin-up, then warm-up and timed launches between HIP events.  GB/s counts",
           "bytes read plus bytes written (copy: 2 x size, the softmax metric's byte count for the same input size).", "",
           "| input size | copy µs | copy GB/s | % of 8 TB/s | read-only GB/s | write-only GB/s |"
           + (" copy µs, trace | read µs, trace | write µs, trace |" if trace else ""),
           "|---|---|---|---|---|---|" + ("---|---|---|" if trace else "")]
    for r in rows:
        line = (f"| {r['mib']} MiB | {r['copy_us']:.2f} | {r['copy_gbps']:.0f} | {100 * r['copy_gbps'] / PEAK_GBPS:.1f} | "
                f"{r['read_gbps']:.0f} | {r['write_gbps']:.0f} |")
        if trace:
            line += "".join(f" {trace[(k, r['mib'])] / 1e3:.2f} |" if (k, r["mib"]) in trace else " |"
                            for k in ("copy16", "read16", "write16"))
        out.append(line)
    if trace:
        out += ["", "The first columns are event-timed in an unprofiled run (the first command).  The trace columns are"
                " kernel durations from a second run under rocprofv3 (the second command), averaged over every dispatch"
                " of that kernel and size (spin-up, warm-up and timed launches); the profiler spaces dispatches out, so"
                " that run's own event timings are not used."]
    path = os.path.join(PROFILE_DIR, "copy_ceiling_sizes.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(open(path).read())


def counter_shapes(keys: list, reps: int = 10) -> list:
    """The dispatch pick of each named workload `reps` times over rotating buffers,
    then a 64 MiB copy kernel to calibrate the byte counters (counter runs)."""
    import torch
    manifest = []
    for key in keys:
        wl = W.WORKLOADS[key]
        res = Resident(wl)
        for i in range(reps):
            res.softmax(i % res.n)
        torch.cuda.synchronize()
        manifest.append({"key": key, "workload": wl.name, "rows": wl.rows, "cols": wl.cols, "dtype": wl.dtype,
                         "kernel": kernel_name(res), "input_bytes": wl.rows * wl.cols * W.elem_size(wl.dtype)})
        log(f"[bench] counters {wl.name}: {reps} launches of {manifest[-1]['kernel']}")
        del res
    n = (64 << 20) // 4
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        binding.bench_copy(a.data_ptr(), b.data_ptr(), n * 4, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return manifest


def summarize_shape_counters(fetch_csv: str, write_csv: str, manifest_json: str) -> None:
    """Write profiles/counters_c5_wide_widths.txt: HBM bytes per dispatch of the dispatch
    pick at each workload of a `bench.py --counter-shapes` run (two rocprofv3 --pmc runs)."""
    manifest = json.load(open(manifest_json))
    tags = {"f32": "F32", "f16": "F16", "bf16": "BF16"}

    def per_group(path, counter):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            wg = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
            d[(name, wg)].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in d.items()}

    fe, wr = per_group(fetch_csv, "FETCH_SIZE"), per_group(write_csv, "WRITE_SIZE")
    cp = next(k for k in fe if "copy16" in k[0])
    cpw = next(k for k in wr if "copy16" in k[0])
    kib = (64 << 20) / 1024
    f_scale, w_scale = kib / fe[cp], kib / wr[cpw]
    rel = lambda f: os.path.relpath(os.path.abspath(f), ROOT)
    keys = ",".join(m["key"] for m in manifest)
    lines = [
        "# HBM traffic of the dispatch pick on the wide c5 sweep widths, MI355X (gfx950)",
        "# Two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE), run from the repository root:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {os.path.dirname(rel(fetch_csv))} -o s -- "
        f"python3 bench.py --counter-shapes {keys} --manifest-out {rel(manifest_json)}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {os.path.dirname(rel(write_csv))} -o s -- "
        f"python3 bench.py --counter-shapes {keys} --manifest-out {rel(manifest_json)}",
        f"# then: python3 bench.py --summarize-shape-counters {rel(fetch_csv)} {rel(write_csv)} {rel(manifest_json)}",
        "# KiB per dispatch averaged over each shape's 10 dispatches (rotating buffers of at least 1 GiB), calibrated",
        f"# with a 64 MiB plain copy of the same run (fetch scale {f_scale:.4f}, write scale {w_scale:.4f}).",
        "# 'x input' divides by the tensor's bytes; a single-pass kernel's ideal is 1.000 for both.",
        f"source_digest: {source_digest()}", ""]
    for m in manifest:
        tag = tags[m["dtype"]]
        hits = [k for k in fe if k[1] == m["rows"] and f"<rws::{tag}," in k[0] and "softmax_" in k[0]]
        if len(hits) != 1:
            lines.append(f"{m['key']}: no unique dispatch group found ({len(hits)} candidates)")
            continue
        k = hits[0]
        fb = fe[k] * f_scale * 1024
        wb = wr.get(k, 0.0) * w_scale * 1024
        size = m["input_bytes"]
        lines.append(f"{m['key']}  [{m['workload']}, {m['kernel']}]")
        lines.append(f"  fetch_bytes: {fb:.0f}  ({fb / size:.4f} x input)")
        lines.append(f"  write_bytes: {wb:.0f}  ({wb / size:.4f} x input)")
        lines.append(f"  traffic_over_algorithmic: {(fb + wb) / (2 * size):.4f}")
    path = os.path.join(PROFILE_DIR, "counters_c5_wide_widths.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def result_line(head: dict, shapes: dict, steps: int, warmup: int, cpu: dict | None, traffic: dict | None) -> dict:
    """The one JSON line: the headline shape's achieved GB/s as `value`, its roofline, the CPU baseline
    and every measured shape."""
    achieved = head["gbps"]
    return {
        "metric": METRIC,
        "value": achieved,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(head["us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(achieved / PAGES_GBPS, 3) if HEADLINE == "c3" else None,
        "dtype": "f32",  # the arithmetic: every kernel widens to fp32 and accumulates there
        "data": "synthetic (seeded N(0,1), resident in HBM, rotating buffers > Infinity Cache)",
        "config": {"workload": head["workload"], "rows": head["rows"], "cols": head["cols"],
                   "storage_dtype": head["dtype"], "accum_dtype": "f32",
                   "kernel": head["kernel"], "buffers": head["buffers"], "peak_gbps": PEAK_GBPS,
                   "copy_kernel_gbps": head.get("copy_kernel_gbps"), "memcpy_gbps": head.get("memcpy_gbps")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": (round(traffic["bytes"]) if traffic else None)},
        "cpu_baseline": cpu,
        "shapes": {k: {kk: vv for kk, vv in v.items() if kk != "_res"} for k, v in shapes.items()},
    }


def wide_only(steps: int, warmup: int) -> dict:
    """The few-wide-rows shapes alone, plus one 64 MiB plain copy to calibrate the byte counters."""
    import torch
    n = (64 << 20) // 4
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        binding.bench_copy(a.data_ptr(), b.data_ptr(), n * 4, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del a, b
    return split_shapes(steps, warmup)


def summarize_wide_counters(fetch_csv, write_csv):
    """Write profiles/counters_wide_rows.txt: HBM bytes per dispatch of the
    one-workgroup-per-row kernel and of the split-row kernels (with a workspace,
    and with the pairs in the output) on the few-wide-rows shapes, from two
    rocprofv3 --pmc runs of `bench.py --wide-only`."""

    def avg(f, counter):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in d.items()}

    fe, wr = avg(fetch_csv, "FETCH_SIZE"), avg(write_csv, "WRITE_SIZE")
    cp = next(k for k in fe if "copy16" in k)
    kib = (64 << 20) / 1024
    f_scale, w_scale = kib / fe[cp], kib / wr[cp]
    tensors = {"F32": ("wide_f32", W.WORKLOADS["wide_f32"]), "BF16": ("wide_bf16", W.WORKLOADS["wide_bf16"])}
    rel = lambda f: os.path.relpath(os.path.abspath(f), ROOT)
    fdir, wdir = os.path.dirname(rel(fetch_csv)), os.path.dirname(rel(write_csv))
    lines = [
        "# HBM traffic of the one-workgroup-per-row kernel and of the split-row kernels on few, wide rows, MI355X (gfx950)",
        "# Two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE), run from the repository root:",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fdir} -o w -- python3 bench.py --wide-only --steps 20 --warmup 5",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {wdir} -o w -- python3 bench.py --wide-only --steps 20 --warmup 5",
        f"# then: python3 bench.py --summarize-wide-counters {rel(fetch_csv)} {rel(write_csv)}",
        "# KiB per dispatch averaged over each kernel's dispatches, calibrated with a 64 MiB plain copy of the same run",
        f"# (fetch scale {f_scale:.4f}, write scale {w_scale:.4f}).  Bytes are per launch, over rotating buffer sets of at",
        "# least 1 GiB, so every launch's first read comes from HBM; 'x input' divides by the tensor's bytes.",
        f"source_digest: {source_digest()}", ""]
    for name in sorted(fe):
        if not any(t in name for t in ("softmax_online", "softmax_row", "softmax_split_")):
            continue
        elem = "BF16" if "BF16" in name else "F32"
        key, wl = tensors[elem]
        size = wl.rows * wl.cols * (4 if elem == "F32" else 2)
        fb, wb = fe[name] * f_scale * 1024, wr.get(name, 0.0) * w_scale * 1024
        lines.append(f"{name[:96]}  [{key} {wl.rows}x{wl.cols}]")
        lines.append(f"  fetch_bytes: {fb:.0f}  ({fb / size:.3f} x input)")
        lines.append(f"  write_bytes: {wb:.0f}  ({wb / size:.3f} x input)")
    path = os.path.join(PROFILE_DIR, "counters_wide_rows.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sweep", action="store_true", help="time every table kernel at every sweep width")
    ap.add_argument("--sweep-out", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None, help="comma-separated workload keys to time (default: c1..c4)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV", default=None,
                    help="write profiles/kernel_trace_bench.md from a rocprofv3 --stats CSV and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/counters_c3_8192x4096_f16.txt from two rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--attention-only", action="store_true",
                    help="time only the attention shapes (and one calibration copy), for counter runs")
    ap.add_argument("--wide-only", action="store_true",
                    help="time only the few-wide-rows shapes (and one calibration copy), for counter runs")
    ap.add_argument("--summarize-wide-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/counters_wide_rows.txt from two rocprofv3 --pmc CSVs of --wide-only")
    ap.add_argument("--summarize-sweep", metavar="SWEEP_JSON", default=None,
                    help="write profiles/sweep_c5_widths.md from a --sweep-out file")
    ap.add_argument("--summarize-attention-counters", nargs="+", metavar="CSV", default=None,
                    help="write profiles/counters_attention_b4_h32_d128_causal.txt from the rocprofv3 --pmc CSVs")
    ap.add_argument("--sweep-keys", default=None,
                    help="with --sweep: comma-separated workload keys to sweep (default: the 24 c5 tensors)")
    ap.add_argument("--copy-sizes", action="store_true",
                    help="time the copy, read-only and write-only streams at 8 MiB ... 1 GiB and exit")
    ap.add_argument("--copy-out", default=None, help="with --copy-sizes: write the table as JSON here")
    ap.add_argument("--summarize-copy-sizes", nargs="+", metavar="JSON [TRACE_CSV]", default=None,
                    help="write profiles/copy_ceiling_sizes.md from a --copy-out file (or a bench JSON line) and,"
                         " optionally, the rocprofv3 kernel-trace CSV of the same run")
    ap.add_argument("--odd-widths", action="store_true",
                    help="time widths that are not a multiple of 16 bytes: the pick, the scalar path, the aligned width")
    ap.add_argument("--odd-out", default=None, help="JSON file for --odd-widths")
    ap.add_argument("--summarize-odd-widths", metavar="JSON", default=None,
                    help="write profiles/odd_widths.md from --odd-widths JSON and exit")
    ap.add_argument("--few-rows", action="store_true",
                    help="time jobs of 256-4096 rows: softmax_fwd and every persistent row shape that fits")
    ap.add_argument("--few-out", default=None, help="JSON file for --few-rows")
    ap.add_argument("--summarize-few-rows", metavar="JSON", default=None,
                    help="write profiles/few_rows_shapes.md from --few-rows JSON and exit")
    ap.add_argument("--ragged-rows", action="store_true",
                    help="time ragged widths (129..255 accesses) at 2 K-64 K rows: the pick and each candidate shape")
    ap.add_argument("--ragged-out", default=None, help="JSON file for --ragged-rows")
    ap.add_argument("--summarize-ragged-rows", metavar="JSON", default=None,
                    help="write profiles/ragged_widths_rows.md from --ragged-rows JSON and exit")
    ap.add_argument("--past-pow2", action="store_true",
                    help="time rows of 300..3800 accesses: the pick and each row shape that holds them")
    ap.add_argument("--past-pow2-out", default=None, help="JSON file for --past-pow2")
    ap.add_argument("--summarize-past-pow2", metavar="JSON", default=None,
                    help="write profiles/past_pow2_widths.md from --past-pow2 JSON and exit")
    ap.add_argument("--split-crossover", action="store_true",
                    help="time one workgroup per row, the split path and softmax_fwd on few, very wide rows")
    ap.add_argument("--split-out", default=None, help="JSON file for --split-crossover")
    ap.add_argument("--summarize-split-crossover", metavar="JSON", default=None,
                    help="write profiles/split_crossover.md from --split-crossover JSON and exit")
    ap.add_argument("--chunk-copy", action="store_true",
                    help="time the chunked copies shaped like the row kernels (192 MiB) and exit")
    ap.add_argument("--chunk-out", default=None, help="with --chunk-copy: write the table as JSON here")
    ap.add_argument("--summarize-chunk-copy", nargs="+", metavar="JSON [BENCH_JSON]", default=None,
                    help="write profiles/chunk_copy_shapes.md from a --chunk-out file (and a default bench line)")
    ap.add_argument("--group-trace", nargs=2, metavar=("TRACE_CSV", "OUT_CSV"), default=None,
                    help="reduce a rocprofv3 kernel trace to per-(kernel, grid) averages and exit")
    ap.add_argument("--counter-shapes", default=None,
                    help="launch the dispatch pick of these workload keys 10 times each, for counter runs")
    ap.add_argument("--manifest-out", default=None, help="with --counter-shapes: write what ran as JSON here")
    ap.add_argument("--summarize-shape-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "MANIFEST_JSON"),
                    default=None, help="write profiles/counters_c5_wide_widths.txt from two --pmc runs")
    ap.add_argument("--no-sweep-widths", action="store_true",
                    help="leave the 24 width-sweep tensors out of the default run")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="leave the copy-ceiling table out of the default run")
    args = ap.parse_args()
    if args.group_trace:
        group_trace(*args.group_trace)
        return 0
    if args.summarize_odd_widths:
        summarize_odd_widths(args.summarize_odd_widths)
        return 0
    if args.summarize_split_crossover:
        summarize_split_crossover(args.summarize_split_crossover)
        return 0
    if args.summarize_few_rows:
        summarize_few_rows(args.summarize_few_rows)
        return 0
    if args.summarize_ragged_rows:
        summarize_ragged_rows(args.summarize_ragged_rows)
        return 0
    if args.summarize_past_pow2:
        summarize_past_pow2(args.summarize_past_pow2)
        return 0
    if args.summarize_chunk_copy:
        summarize_chunk_copy(*args.summarize_chunk_copy[:2])
        return 0
    if args.summarize_copy_sizes:
        summarize_copy_sizes(*args.summarize_copy_sizes[:2])
        return 0
    if args.summarize_shape_counters:
        summarize_shape_counters(*args.summarize_shape_counters)
        return 0
    if args.summarize_attention_counters:
        summarize_attention_counters(args.summarize_attention_counters)
        return 0

    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep)
        return 0
    if args.summarize_wide_counters:
        summarize_wide_counters(*args.summarize_wide_counters)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return 0

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); rows of a softmax "
              "are independent, so a multi-GPU run would be one independent launch per GPU shard.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    binding._load()
    log(f"[bench] {binding.version()} on {torch.cuda.get_device_name(0)}")

    if args.attention_only:
        print(json.dumps(attention_only(args.steps, args.warmup)), flush=True)
        return 0
    if args.wide_only:
        print(json.dumps(wide_only(args.steps, args.warmup)), flush=True)
        return 0
    if args.sweep:
        out = sweep(args.steps, args.warmup, args.sweep_keys.split(",") if args.sweep_keys else None)
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                json.dump(out, f, indent=1)
        return 0
    if args.copy_sizes:
        table = copy_ceiling(args.steps, args.warmup)
        if args.copy_out:
            with open(args.copy_out, "w") as f:
                json.dump(table, f, indent=1)
        print(json.dumps(table), flush=True)
        return 0
    if args.odd_widths:
        table = odd_widths(args.steps, args.warmup)
        if args.odd_out:
            with open(args.odd_out, "w") as f:
                json.dump(table, f, indent=1)
        return 0
    if args.few_rows:
        table = few_rows(args.steps, args.warmup)
        if args.few_out:
            with open(args.few_out, "w") as f:
                json.dump(table, f, indent=1)
        return 0
    if args.past_pow2:
        table = past_pow2(args.steps, args.warmup)
        if args.past_pow2_out:
            with open(args.past_pow2_out, "w") as f:
                json.dump(table, f, indent=1)
        return 0
    if args.ragged_rows:
        table = ragged_rows(args.steps, args.warmup)
        if args.ragged_out:
            with open(args.ragged_out, "w") as f:
                json.dump(table, f, indent=1)
        return 0
    if args.split_crossover:
        table = split_crossover(args.steps, args.warmup)
        if args.split_out:
            with open(args.split_out, "w") as f:
                json.dump(table, f, indent=1)
        return 0
    if args.chunk_copy:
        table = chunk_copy(args.steps, args.warmup)
        if args.chunk_out:
            with open(args.chunk_out, "w") as f:
                json.dump(table, f, indent=1)
        print(json.dumps(table), flush=True)
        return 0
    if args.counter_shapes:
        manifest = counter_shapes(args.counter_shapes.split(","))
        if args.manifest_out:
            with open(args.manifest_out, "w") as f:
                json.dump(manifest, f, indent=1)
        print(json.dumps(manifest), flush=True)
        return 0

    keys = args.only.split(",") if args.only else FIXED
    if HEADLINE not in keys:
        keys = [HEADLINE] + keys
    shapes = {}
    for key in keys:
        shapes[key] = measure_shape(key, args.steps, args.warmup, with_copy=True, with_unfused=key in ("c3", "c4"))
        if key != HEADLINE:
            del shapes[key]["_res"]  # free its buffers before the next shape
    copy_table = None
    if args.only is None:
        shapes["c2_fused"] = causal_c2(args.steps, args.warmup)
        shapes.update(split_shapes(args.steps, args.warmup))
        shapes.update(attention_shapes(args.steps, args.warmup))
        if not args.no_sweep_widths:
            for dt in ("bf16", "f32"):
                for w in W.SWEEP_WIDTHS:
                    key = f"c5_{dt}_{w}"
                    shapes[key] = measure_shape(key, args.steps, args.warmup, with_copy=True, light=True)
                    del shapes[key]["_res"]
        if not args.no_copy_ceiling:
            copy_table = copy_ceiling(args.steps, args.warmup)

    head = shapes[HEADLINE]
    res = head.pop("_res")
    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu baseline: oracle on {head['workload']} for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(res, args.cpu_seconds)
    info = next(k for k in binding.kernel_table() if k.name == head["kernel"])
    line = result_line(head, shapes, args.steps, args.warmup, cpu, stored_traffic(head["workload"], info))
    if copy_table is not None:
        line["copy_ceiling"] = copy_table
    wide = [v for k, v in shapes.items() if k.startswith("c5_") and v["cols"] >= 2048]
    if wide:
        line["sweep_widths_ge_2048"] = {
            "min_frac_of_peak": min(v["frac_of_peak"] for v in wide),
            "at_or_above_0.8": sum(v["frac_of_peak"] >= 0.8 for v in wide), "of": len(wide)}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
