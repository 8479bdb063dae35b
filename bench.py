#!/usr/bin/env python3
"""Throughput of the row-wise kernels on one MI355X.

One step = one call of the hot path on one batch of the headline workload:
fused LayerNorm + affine + tanh GeLU, fp32, x[4096, 768] ~ N(0,1),
w = 1 + 0.1 N(0,1), b = 0.1 N(0,1), eps = 1e-5.  Inputs are resident in HBM
before the timed region; consecutive steps rotate over >= 1 GiB of distinct
input/output buffers so that the 256 MB memory-side cache cannot serve them.

Prints one JSON line.  `value` is achieved HBM GB/s on the algorithmic bytes
(one read of x, w and b, one write of y) over the wall-clock time of K steps
bracketed by device synchronizations.  The K steps are launched as one HIP
graph (captured before the timed region; `--launch stream` launches them one
by one from Python instead, where the host's launch rate, not the GPU, sets
the pace of a 5 us kernel).  `roofline.achieved` divides the same bytes by the
kernel's average per-dispatch device time in the committed rocprofv3 kernel
trace of this command (profiles/kernel_trace_all_cases.txt), the basis the
70% bar is judged on; the live HIP-event rate of back-to-back launches on the
kernel's stream is reported beside it (`achieved_live_events`).
`detail` holds the same measurement for every other workload (softmax fp32
8192x1000, online softmax fp32 64x262144 streaming and split-row, bf16
16384x4096 LayerNorm+GeLU and softmax, long-row LayerNorm streaming and split,
row sum and max, elementwise GeLU, RMSNorm and fused residual RMSNorm, and the
flash-attention forward in TFLOP/s against the 2.5 PFLOP/s matrix-core peak)
and the 16-byte copy ceiling.
`cpu_baseline` is the CPU oracle timed on this host on repeated full batches.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix cores, published
ROTATE_BYTES = 1 << 30
EPS = 1e-5
METRIC = "achieved HBM GB/s (% of MI355X peak) and rows/s for softmax & LayerNorm+GeLU"
HEADLINE = "ln_gelu_f32_4096x768"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- cases


class Case:
    """One kernel on one workload, with rotating buffer sets and a raw launch."""

    def __init__(self, name, op, workload, splits=None, rows=None, passes=2):
        self.name, self.op, self.workload, self.splits = name, op, workload, splits
        self.rows = rows
        # passes over the rows: 2 for a row held on chip (one read, one
        # write), 3 for rows read twice (the long rows of the split form)
        self.passes = passes

    def setup(self, torch, rk, rowgen):
        d = rowgen.make(self.workload)
        norm = self.op in ("layernorm_gelu", "layernorm_gelu_ex", "rmsnorm", "residual_rmsnorm")
        x = d["x"] if norm else d["x_softmax"]
        M, N = x.shape
        es = x.element_size()
        self.M, self.N, self.dtype = M, N, x.dtype
        self.dtype_code = rk.RK_F32 if x.dtype == torch.float32 else rk.RK_BF16
        io = 2 * M * N * es
        footprint = io
        if self.op == "layernorm_gelu":
            self.bytes = self.passes * M * N * es + 2 * N * es  # x, y, and w, b once
        elif self.op == "layernorm_gelu_ex":
            if self.splits == 0:
                self.splits = rk.rk_layernorm_gelu_auto_splits(M, N, self.dtype_code)
            # two reads of x, one write of y, w and b once (+ partials out and in)
            self.bytes = 3 * M * N * es + 2 * N * es
            if self.splits > 1:
                self.bytes += 2 * M * self.splits * 8
        elif self.op in ("row_sum", "row_max"):
            self.bytes = M * N * es + M * es  # one read of x, M results
            footprint = M * N * es
        elif self.op == "row_sum_ex":
            if self.splits == 0:
                self.splits = rk.rk_row_reduce_auto_splits(M, N, self.dtype_code)
            # one read of x, M results (+ one float per chunk out and in)
            self.bytes = M * N * es + M * es
            if self.splits > 1:
                self.bytes += 2 * M * self.splits * 4
            footprint = M * N * es
        elif self.op == "rmsnorm":
            self.bytes = io + N * es  # x, y, and w once
        elif self.op == "residual_rmsnorm":
            self.bytes = 2 * io + N * es  # x, residual, y, residual_out, and w once
            footprint = 2 * io
        elif self.op == "online" and self.splits == 1:
            self.bytes = 3 * M * N * es  # two reads of x, one write
        elif self.op == "online":
            if self.splits == 0:
                self.splits = rk.rk_online_softmax_auto_splits(M, N, self.dtype_code)
            self.bytes = 3 * M * N * es + 2 * M * self.splits * 8  # + partials out and in
        else:
            self.bytes = self.passes * M * N * es
        self.R = max(2, math.ceil(ROTATE_BYTES / footprint))
        dev = torch.device("cuda")
        xd = x.to(dev)
        self.xs = [xd] + [xd.clone() for _ in range(self.R - 1)]
        self.ys = [torch.empty_like(xd) for _ in range(self.R)]
        if self.op == "residual_rmsnorm":
            rd = rowgen.residual(self.workload).to(dev)
            self.rs = [rd] + [rd.clone() for _ in range(self.R - 1)]
            self.ros = [torch.empty_like(xd) for _ in range(self.R)]
        self.w = d["w"].to(dev)
        self.b = d["b"].to(dev)
        self.ws = None
        if self.op == "online" and self.splits > 1:
            nb = rk.rk_online_softmax_workspace_bytes(M, N, self.splits, self.dtype_code)
            self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        if self.op == "layernorm_gelu_ex" and self.splits > 1:
            nb = rk.rk_layernorm_gelu_workspace_bytes(M, N, self.splits, self.dtype_code)
            self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        if self.op == "row_sum_ex" and self.splits > 1:
            nb = rk.rk_row_reduce_workspace_bytes(M, N, self.splits, self.dtype_code)
            self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        lib = rk.load()
        stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        fp = ctypes.c_float(EPS)
        if self.op == "layernorm_gelu":
            fn = lib.rk_layernorm_gelu
            self.args = [(xx.data_ptr(), self.w.data_ptr(), self.b.data_ptr(), yy.data_ptr(), M,
                          N, N, N, fp, self.dtype_code, stream)
                         for xx, yy in zip(self.xs, self.ys)]
        elif self.op == "layernorm_gelu_ex":
            fn = lib.rk_layernorm_gelu_ex
            wp = self.ws.data_ptr() if self.ws is not None else None
            wb = self.ws.numel() if self.ws is not None else 0
            self.args = [(xx.data_ptr(), self.w.data_ptr(), self.b.data_ptr(), yy.data_ptr(), M,
                          N, N, N, fp, self.dtype_code, 0, self.splits, wp, wb, stream)
                         for xx, yy in zip(self.xs, self.ys)]
        elif self.op in ("row_sum", "row_max"):
            fn = getattr(lib, "rk_" + self.op)
            self.ys = [torch.empty(M, dtype=x.dtype, device=dev) for _ in range(self.R)]
            self.args = [(xx.data_ptr(), yy.data_ptr(), M, N, N, self.dtype_code, stream)
                         for xx, yy in zip(self.xs, self.ys)]
        elif self.op == "row_sum_ex":
            fn = lib.rk_row_sum_ex
            wp = self.ws.data_ptr() if self.ws is not None else None
            wb = self.ws.numel() if self.ws is not None else 0
            self.ys = [torch.empty(M, dtype=x.dtype, device=dev) for _ in range(self.R)]
            self.args = [(xx.data_ptr(), yy.data_ptr(), M, N, N, self.dtype_code, self.splits,
                          wp, wb, stream) for xx, yy in zip(self.xs, self.ys)]
        elif self.op == "gelu":
            fn = lib.rk_gelu
            self.args = [(xx.data_ptr(), yy.data_ptr(), M, N, N, N, self.dtype_code, 0, stream)
                         for xx, yy in zip(self.xs, self.ys)]
        elif self.op == "rmsnorm":
            fn = lib.rk_rmsnorm
            self.args = [(xx.data_ptr(), self.w.data_ptr(), yy.data_ptr(), M, N, N, N, fp,
                          self.dtype_code, stream) for xx, yy in zip(self.xs, self.ys)]
        elif self.op == "residual_rmsnorm":
            fn = lib.rk_residual_rmsnorm
            self.args = [(xx.data_ptr(), rr.data_ptr(), self.w.data_ptr(), yy.data_ptr(),
                          oo.data_ptr(), M, N, N, N, N, N, fp, self.dtype_code, stream)
                         for xx, rr, yy, oo in zip(self.xs, self.rs, self.ys, self.ros)]
        elif self.op == "softmax":
            fn = lib.rk_softmax
            self.args = [(xx.data_ptr(), yy.data_ptr(), M, N, N, N, self.dtype_code, stream)
                         for xx, yy in zip(self.xs, self.ys)]
        else:
            fn = lib.rk_online_softmax
            wp = self.ws.data_ptr() if self.ws is not None else None
            wb = self.ws.numel() if self.ws is not None else 0
            self.args = [(xx.data_ptr(), yy.data_ptr(), M, N, N, N, self.dtype_code, self.splits,
                          wp, wb, stream) for xx, yy in zip(self.xs, self.ys)]
        self.fn = fn
        return self

    def launch(self, i):
        st = self.fn(*self.args[i % self.R])
        if st != 0:
            raise RuntimeError(f"{self.name}: status {st}")

    def rebind(self, stream):
        """Launch on `stream` from now on (the stream is every entry point's
        last argument)."""
        self.args = [a[:-1] + (stream,) for a in self.args]

    def free(self):
        self.xs = self.ys = self.args = self.ws = None
        self.rs = self.ros = None


class AttnCase:
    """rk_flash_attention on [B, H, T, d] inputs: MFMA-bound, reported in
    TFLOP/s (4 B H T^2 d flops, about half of that causal: 2 B H T (T+1) d)."""

    def __init__(self, name, B, H, T, d, dtype, causal):
        self.name, self.B, self.H, self.T, self.d = name, B, H, T, d
        self.dtype_name, self.causal = dtype, causal

    def setup(self, torch, rk, rowgen):
        dt = {"bf16": torch.bfloat16, "f16": torch.float16}[self.dtype_name]
        B, H, T, d = self.B, self.H, self.T, self.d
        q, k, v = rowgen.attention_qkv(B, H, T, d, dt, seed=3000 + T)
        dev = torch.device("cuda")
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.o = torch.empty_like(self.q)
        self.M = None
        self.flops = (2.0 * B * H * T * (T + 1) * d if self.causal else 4.0 * B * H * T * T * d)
        self.bytes = 4 * B * H * T * d * q.element_size()  # q, k, v read once, o written
        self.R = 1  # compute-bound: no buffer rotation needed
        lib = rk.load()
        self.fn = lib.rk_flash_attention
        code = rk.RK_BF16 if dt == torch.bfloat16 else rk.RK_F16
        stream = torch.cuda.current_stream().cuda_stream
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                     B, H, T, d, None, None, None, None, ctypes.c_float(1.0 / math.sqrt(d)),
                     int(self.causal), code, stream)
        return self

    def launch(self, i):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"{self.name}: status {st}")

    def free(self):
        self.q = self.k = self.v = self.o = self.args = None


class CopyCase:
    """The 16-byte copy kernel: achievable read+write bandwidth."""

    def __init__(self, name, nbytes, max_wg=0):
        self.name, self.nbytes, self.max_wg = name, nbytes, max_wg

    def setup(self, torch, rk, rowgen):
        dev = torch.device("cuda")
        self.bytes = 2 * self.nbytes
        self.R = max(2, math.ceil(ROTATE_BYTES / self.bytes))
        self.M = None
        self.src = [torch.full((self.nbytes // 4,), 1.0, device=dev) for _ in range(self.R)]
        self.dst = [torch.empty_like(s) for s in self.src]
        lib = rk.load()
        self.fn = lib.rk_probe_copy
        stream = torch.cuda.current_stream().cuda_stream
        self.args = [(s.data_ptr(), d.data_ptr(), self.nbytes, self.max_wg, stream)
                     for s, d in zip(self.src, self.dst)]
        return self

    def launch(self, i):
        st = self.fn(*self.args[i % self.R])
        if st != 0:
            raise RuntimeError(f"{self.name}: status {st}")

    def free(self):
        self.src = self.dst = self.args = None


def all_cases():
    return [
        Case("ln_gelu_f32_4096x768", "layernorm_gelu", "ln_gelu_f32_4096x768"),
        Case("softmax_f32_8192x1000", "softmax", "softmax_f32_8192x1000"),
        Case("online_stream_f32_64x262144", "online", "online_f32_64x262144", splits=1),
        Case("online_split64_f32_64x262144", "online", "online_f32_64x262144", splits=64),
        Case("online_auto_f32_64x262144", "online", "online_f32_64x262144", splits=0),
        Case("ln_gelu_bf16_16384x4096", "layernorm_gelu", "bf16_16384x4096"),
        Case("softmax_bf16_16384x4096", "softmax", "bf16_16384x4096"),
        Case("ln_gelu_stream_f32_64x262144", "layernorm_gelu_ex", "ln_long_f32_64x262144",
             splits=1),
        Case("ln_gelu_split64_f32_64x262144", "layernorm_gelu_ex", "ln_long_f32_64x262144",
             splits=64),
        Case("ln_gelu_auto_f32_64x262144", "layernorm_gelu_ex", "ln_long_f32_64x262144",
             splits=0),
        # the same long rows through the entry points that take no workspace
        # (split with the partials kept in the output: two reads, one write)
        Case("softmax_f32_64x262144", "softmax", "online_f32_64x262144", passes=3),
        Case("ln_gelu_f32_64x262144", "layernorm_gelu", "ln_long_f32_64x262144", passes=3),
        Case("row_sum_f32_8192x1000", "row_sum", "softmax_f32_8192x1000"),
        Case("row_max_f32_8192x1000", "row_max", "softmax_f32_8192x1000"),
        Case("row_sum_f32_64x262144", "row_sum", "online_f32_64x262144"),
        Case("row_sum_split_f32_64x262144", "row_sum_ex", "online_f32_64x262144", splits=0),
        Case("row_sum_bf16_16384x4096", "row_sum", "bf16_16384x4096"),
        Case("gelu_bf16_16384x4096", "gelu", "bf16_16384x4096"),
        Case("rmsnorm_f32_4096x768", "rmsnorm", "ln_gelu_f32_4096x768"),
        Case("residual_rmsnorm_f32_4096x768", "residual_rmsnorm", "ln_gelu_f32_4096x768"),
        Case("rmsnorm_bf16_16384x4096", "rmsnorm", "bf16_16384x4096"),
        Case("residual_rmsnorm_bf16_16384x4096", "residual_rmsnorm", "bf16_16384x4096"),
        AttnCase("attn_bf16_1x8x4096x128", 1, 8, 4096, 128, "bf16", False),
        AttnCase("attn_bf16_4x32x1024x128", 4, 32, 1024, 128, "bf16", False),
        AttnCase("attn_bf16_4x32x4096x128", 4, 32, 4096, 128, "bf16", False),
        AttnCase("attn_causal_bf16_4x32x4096x128", 4, 32, 4096, 128, "bf16", True),
        AttnCase("attn_f16_4x32x4096x128", 4, 32, 4096, 128, "f16", False),
        CopyCase("copy_256MiB", 256 << 20),
        # copies of the same total traffic as the small workloads: the
        # achievable ceiling at that size (launch and latency included)
        CopyCase("copy_12MiB", 12 << 20),
        CopyCase("copy_32MiB", 32 << 20),
        CopyCase("copy_64MiB_64wg", 64 << 20, max_wg=64),
    ]


# --------------------------------------------------------------- timing


def event_time(torch, case, K, W, reps=3, spread=None):
    """Median over `reps` of (elapsed of K back-to-back launches) / K, in s
    (`spread`, if a dict, receives the minimum and maximum)."""
    for i in range(W):
        case.launch(i)
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(K):
            case.launch(i)
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e) * 1e-3 / K)
    if spread is not None:
        spread["min"], spread["max"] = min(out), max(out)
    return statistics.median(out)


def wall_time(torch, case, K, W, graph):
    """Headline protocol: W untimed steps, then exactly K steps bracketed by
    device synchronizations; returns the wall seconds of the K steps.
    With `graph`, the K steps (each on its own rotation set) are captured
    into one HIP graph after the warmup, and the timed region is one replay
    of it."""
    for i in range(W):
        case.launch(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            case.rebind(torch.cuda.current_stream().cuda_stream)
            for i in range(K):
                case.launch(W + i)
        case.rebind(torch.cuda.current_stream().cuda_stream)
        # upload the executable graph now, so that the timed replay does not
        # pay for it (measured 7.5 -> 6.6 us per step over 20 steps)
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if hip.hipGraphUpload(g.raw_cuda_graph_exec(), torch.cuda.current_stream().cuda_stream):
            log("hipGraphUpload failed: the timed replay includes the upload")
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if g is not None:
        g.replay()
    else:
        for i in range(K):
            case.launch(W + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0


def head_kernel_name(rk, N):
    i = rk.variant_pick(rk.RK_OP_LAYERNORM_GELU, rk.RK_F32, N)
    v = rk.variants(rk.RK_OP_LAYERNORM_GELU, rk.RK_F32)[i]
    return ("layernorm_gelu_tile<float, G={waves_per_row}, V={vecs_per_lane}, "
            "W={waves_per_block}, R={rows_per_group}>".format(**v))


# ------------------------------------------------------- counters / cpu


def code_tokens(text):
    """C++ source with comments and whitespace removed (string literals kept):
    a comment-only edit leaves the compiled kernel, and this, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif c.isspace():
            i += 1
        else:
            out.append(c)
            i += 1
    return "".join(out)


def kernel_source_hash():
    """Hash of the headline kernel's sources, comments and whitespace aside."""
    h = hashlib.sha256()
    for f in ("rk_layernorm_gelu.hip", "rk_device.h"):
        with open(os.path.join(ROOT, "row_wise_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(case_name):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when it is missing or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{case_name}.txt")
    if not os.path.exists(path):
        return None
    m = re.search(r"^TRAFFIC (\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def profiled_duration(case_name):
    """(avg, median) per-dispatch duration in us of the case's kernel in the
    committed rocprofv3 kernel trace, or None when it is missing or was taken
    of other kernel sources."""
    path = os.path.join(ROOT, "profiles", "kernel_trace_all_cases.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_source_sha (\w+)\s*$", text, flags=re.M)
    if not m or m.group(1) != kernel_source_hash():
        return None
    for line in text.splitlines():
        f = line.split()
        if len(f) >= 12 and f[0] == case_name:
            return float(f[8]), float(f[9])
    return None


def cpu_baseline(seconds):
    import numpy as np

    import oracle
    import rowgen

    d = rowgen.make(HEADLINE)
    x, w, b = (d[k].double().numpy() for k in ("x", "w", "b"))
    M, N = x.shape
    nbytes = 2 * M * N * 4 + 2 * N * 4
    orc = oracle.default()
    eps = float(np.float32(EPS))
    orc.layernorm_gelu(x[:16], w, b, eps)  # load / warm

    def timed(fn, budget):
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return passes, el

    # one thread on whole batches
    passes, el = timed(lambda: orc.layernorm_gelu(x, w, b, eps), seconds)
    # the same oracle on every core of this process's affinity mask, one row
    # block per thread (the C call releases the interpreter lock)
    from concurrent.futures import ThreadPoolExecutor

    # (at most 16 threads: the CPU share that one GPU's host process gets)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    blocks = [x[i * M // cores:(i + 1) * M // cores] for i in range(cores)]
    with ThreadPoolExecutor(cores) as pool:
        def batch():
            list(pool.map(lambda blk: orc.layernorm_gelu(blk, w, b, eps), blocks))
        p_n, el_n = timed(batch, seconds / 2)
    return {
        "value": round(passes * nbytes / el / 1e9, 4),
        "unit": "GB/s",
        "rows_per_s": round(passes * M / el, 1),
        "cores": 1,
        "kind": "oracle",
        "sample": f"full {M}x{N} fp32 batch, {passes} passes in {el:.1f} s, single thread, "
                  f"double precision",
        "all_cores": {"value": round(p_n * nbytes / el_n / 1e9, 4), "unit": "GB/s",
                      "rows_per_s": round(p_n * M / el_n, 1), "cores": cores,
                      "sample": f"{p_n} full batches in {el_n:.1f} s, {cores} threads over row "
                                f"blocks"},
        "cpu": cpu_model(),
    }


def cpu_model():
    """The host CPU's model name as lscpu prints it (else /proc/cpuinfo), with
    lscpu's CPU family, model and stepping (a virtualised host may report only
    a generic name such as "AMD EPYC")."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        fields = {}
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
        if "Model name" in fields:
            ids = [f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping") if k in fields]
            return fields["Model name"] + (f" ({', '.join(ids)})" if ids else "")
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ main


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--case", default=None, help="time only this case (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--launch", choices=("graph", "stream"), default="graph",
                    help="headline timed region: one HIP graph of the K steps, or K launches")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (rows "
              "would shard across GPUs by row blocks, with no communication)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    import torch

    import row_wise_amd as rk
    import rowgen

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    rk.load()
    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup

    cases = all_cases()
    if args.case:
        cases = [c for c in cases if c.name == args.case]
        if not cases:
            sys.exit(f"unknown case {args.case}")

    detail = []
    head = None
    for c in cases:
        log(f"case {c.name}: setup")
        c.setup(torch, rk, rowgen)
        spread = {}
        if c.name == HEADLINE:
            wall = wall_time(torch, c, K, W, args.launch == "graph")
            t_evt = event_time(torch, c, K, W)
            head = (c, wall, t_evt)
            t = t_evt
        else:
            t = event_time(torch, c, K, W, spread=spread)
        rec = {"case": c.name, "us_per_call": round(t * 1e6, 3),
               "GB_per_s": round(c.bytes / t / 1e9, 1),
               "pct_hbm_peak": round(100 * c.bytes / t / 1e9 / HBM_PEAK_GBS, 1),
               "bytes_per_call": c.bytes, "rotation_sets": c.R}
        if getattr(c, "flops", None):
            rec["TFLOP_per_s"] = round(c.flops / t / 1e12, 1)
            rec["pct_mfma_peak"] = round(100 * c.flops / t / 1e12 / MFMA_PEAK_TFLOPS, 1)
        if c.M is not None:
            rec["rows_per_s"] = round(c.M / t, 1)
        if getattr(c, "splits", None):
            rec["splits"] = c.splits
        if c.name != HEADLINE and spread:
            rec["us_min_max"] = [round(spread["min"] * 1e6, 3), round(spread["max"] * 1e6, 3)]
        if getattr(c, "op", None) in ("online", "layernorm_gelu_ex") or getattr(c, "passes", 2) == 3:
            # against the one-read-one-write minimum (the row cannot stay on chip)
            rec["GB_per_s_1R1W"] = round(2 * c.M * c.N * (4 if c.dtype_code == 0 else 2) / t / 1e9, 1)
        detail.append(rec)
        if "TFLOP_per_s" in rec:
            log(f"case {c.name}: {rec['us_per_call']} us  {rec['TFLOP_per_s']} TFLOP/s "
                f"({rec['pct_mfma_peak']}% of 2.5 PFLOP/s)")
        else:
            log(f"case {c.name}: {rec['us_per_call']} us  {rec['GB_per_s']} GB/s "
                f"({rec['pct_hbm_peak']}% of 8 TB/s)")
        c.free()
        torch.cuda.empty_cache()

    if head is None:
        print(json.dumps({"detail": detail}))
        return

    c, wall, t_evt = head
    value = c.bytes * K / wall / 1e9
    live = c.bytes / t_evt / 1e9
    # device time per dispatch from the committed trace of this command (the
    # basis of the bar); the live event rate when no current trace exists
    prof = profiled_duration(c.name)
    achieved = c.bytes / (prof[0] * 1e-6) / 1e9 if prof is not None else live
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "op": "fused LayerNorm+affine+tanh-GeLU",
                   "M": c.M, "N": c.N, "dtype": "f32", "eps": EPS,
                   "bytes_per_step": c.bytes, "rotation_sets": c.R,
                   "launch": "one HIP graph of the K steps" if args.launch == "graph"
                   else "K launches from the host"},
        "rows_per_s": round(c.M * K / wall, 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(c.name),
            "kernel": head_kernel_name(rk, c.N),
            "basis": ("average per-dispatch device time in profiles/kernel_trace_all_cases.txt"
                      if prof is not None else "live HIP events (no trace of these sources)"),
            "us_per_launch_trace_avg_median": list(prof) if prof is not None else None,
            "achieved_live_events": round(live, 2),
            "frac_live_events": round(live / HBM_PEAK_GBS, 4),
            "us_per_launch_live_events": round(t_evt * 1e6, 3),
        },
        "detail": detail,
    }
    if not args.no_cpu:
        log("cpu baseline: oracle on the host")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
