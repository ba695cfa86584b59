"""Benchmark of the block-FP8 decode GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the decode and speculative-verify shapes M = 1..8 on the largest
logged weight shape N = 17408, K = 5120 (page 2, ownding.com L20 report,
section 8). One step is one pass of the whole hot path over that workload:
for every M, the per-token activation quantisation and the block-FP8 GEMM,
run as one launch (fp8bq_gemm_fused, bitwise the result of fp8bq_quant_act
followed by fp8bq_gemm). The two-call form and the weight-only path
(fp8bq_gemm_w8a16) are timed on the same workload beside it. Inputs are
resident in HBM before timing. The weights rotate over enough distinct
copies (>= 1 GiB) that no call finds its 89 MB weight in the 256 MB
Infinity Cache, so every GEMM reads W from HBM.

Printed: one JSON line with the step throughput (algorithmic bytes per step
/ step time, GB/s), per-M microseconds per call from HIP events on the
launch stream, the roofline of the dominant kernel (the GEMM), the prefill
GEMMs (M = 3465) against the FP8 MFMA peak, two-stage vocabulary scoring
(coarse FP8 logits, exact top-64, exact bf16 rescoring; V = 152064 stand-in,
K = 5120) per stage and per M, and the CPU oracle timed on a bounded sample
of the same workload.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import memory_bound_w8a8_amd as fp8bq  # noqa: E402
import workloads  # noqa: E402

N, K = 17408, 5120
MS = list(range(1, 9))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MALL_BYTES = 256 << 20
METRIC = "block-FP8 GEMM HBM GB/s (% of peak) + us/call, M=1-8, N=17408 K=5120"


def gemm_bytes(m, n, k):
    """Algorithmic bytes of one GEMM call: W codes + W scales + A codes +
    A scales + C (bf16)."""
    g = k // 128
    return n * k + 4 * ((n + 127) // 128) * g + m * k + 4 * m * g + 2 * m * n


def quant_bytes(m, k):
    """Algorithmic bytes of one activation quantisation: bf16 in, codes and
    fp32 scales out."""
    return 2 * m * k + m * k + 4 * m * (k // 128)


def bf16_act_bytes(m, n, k):
    """Algorithmic bytes of one call that takes the bf16 activation (fused
    or weight-only): W codes + W scales + bf16 activation + C (bf16)."""
    g = k // 128
    return n * k + 4 * ((n + 127) // 128) * g + 2 * m * k + 2 * m * n


def kernel_source_digest():
    """Hash of the sources that define the dominant kernel (the row-range
    streaming GEMM and its launch configuration), to tie stored counter data
    to the code it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_bound_w8a8_amd", "csrc")
    for f in ("device_common.h", "gemm_rows.h", "rows_launch.h", "gemm_fused.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(digest):
    """HBM traffic per GEMM launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "gemm_rows_fused_decode_M1-8_N17408_K5120_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                key, _, val = ln.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_digest") != digest:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Plan:
    """Device buffers and raw C-ABI launch arguments for one step."""

    def __init__(self, copies, seed=1234):
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(self.dev)
        self.lib = fp8bq.lib()
        g = torch.Generator(device=self.dev)
        self.w = []
        for i in range(copies):
            g.manual_seed(seed + i)
            w32 = torch.randn((N, K), generator=g, device=self.dev, dtype=torch.float32).mul_(0.02)
            self.w.append(fp8bq.quant_weight(w32))
            del w32
        self.a = {m: workloads.activation(m, N, K).to(self.dev) for m in MS}
        self.aq = {m: torch.empty((m, K), dtype=torch.uint8, device=self.dev) for m in MS}
        self.as_ = {m: torch.empty((m, K // 128), dtype=torch.float32, device=self.dev) for m in MS}
        self.c = {m: torch.empty((m, N), dtype=torch.bfloat16, device=self.dev) for m in MS}
        self.s = ctypes.c_void_p(self.stream.cuda_stream)
        self.next_w = 0
        torch.cuda.synchronize()

    def quant(self, m):
        st = self.lib.fp8bq_quant_act(m, K, self.a[m].data_ptr(), self.aq[m].data_ptr(), self.as_[m].data_ptr(),
                                      self.s)
        if st:
            raise fp8bq.Fp8bqError("fp8bq_quant_act", st)

    def gemm(self, m):
        wq, ws = self.w[self.next_w]
        self.next_w = (self.next_w + 1) % len(self.w)
        st = self.lib.fp8bq_gemm(m, N, K, self.aq[m].data_ptr(), self.as_[m].data_ptr(), wq.data_ptr(),
                                 ws.data_ptr(), self.c[m].data_ptr(), self.s)
        if st:
            raise fp8bq.Fp8bqError("fp8bq_gemm", st)

    def w8a16(self, m):
        wq, ws = self.w[self.next_w]
        self.next_w = (self.next_w + 1) % len(self.w)
        st = self.lib.fp8bq_gemm_w8a16(m, N, K, self.a[m].data_ptr(), wq.data_ptr(), ws.data_ptr(),
                                       self.c[m].data_ptr(), self.s)
        if st:
            raise fp8bq.Fp8bqError("fp8bq_gemm_w8a16", st)

    def step(self):
        for m in MS:
            self.quant(m)
            self.gemm(m)

    def fused(self, m):
        wq, ws = self.w[self.next_w]
        self.next_w = (self.next_w + 1) % len(self.w)
        st = self.lib.fp8bq_gemm_fused(m, N, K, self.a[m].data_ptr(), wq.data_ptr(), ws.data_ptr(),
                                       self.c[m].data_ptr(), self.s)
        if st:
            raise fp8bq.Fp8bqError("fp8bq_gemm_fused", st)

    def step_fused(self):
        for m in MS:
            self.fused(m)

    def step_w8a16(self):
        for m in MS:
            self.w8a16(m)


def time_kernels(plan, reps):
    """Average duration of each launch kind, from HIP events on the launch
    stream around `reps` back-to-back launches (rotating weights)."""
    out = {}
    for m in MS:
        for kind, fn in (("gemm", plan.gemm), ("quant", plan.quant), ("w8a16", plan.w8a16), ("fused", plan.fused)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            fn(m)
            e0.record(plan.stream)
            for _ in range(reps):
                fn(m)
            e1.record(plan.stream)
            e1.synchronize()
            out[(kind, m)] = e0.elapsed_time(e1) * 1e3 / reps  # us
    return out


FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA


def scaled_mfma_tflops(dev, grid=1024, iters=4096):
    """FP8 16x16x128 MFMA rate of the block-scaled GEMM's inner loop (fresh
    products, 4 fp32 scale FMAs per MFMA) on quantised Gaussian codes: the
    most a GEMM that scales each group's products gets from the matrix
    cores on this GPU."""
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    vals = torch.randn(fp8bq.MB_MFMA_DATA_BYTES, generator=g, device=dev).mul_(448.0 / 4.0)
    codes = vals.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    us = graph_us(lambda i: fp8bq.mb_mfma_scaled(grid, iters, codes, 0.5, sink=sink), 3)
    return grid * 4 * 8 * iters * 2.0 * 16 * 16 * 128 / us / 1e6


def prefill(plan, reps=20):
    """Prefill GEMMs (M = 3465 tokens, page 2 section 4.2) on the two logged
    shapes that take it, timed with HIP events on the launch stream around
    three windows of `reps` back-to-back calls after a warm-up window (the
    median window is reported): the compute-bound (MFMA) regime of the same
    entry point. Weights and activations are synthetic and resident."""
    dev = plan.dev
    m = workloads.PREFILL_M
    out = []
    scaled_loop = scaled_mfma_tflops(dev)
    g = torch.Generator(device=dev)
    for n, k in workloads.PREFILL_SHAPES:
        if (n, k) == (N, K):
            wq, ws = plan.w[0]
        else:
            g.manual_seed(99)
            w32 = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
            wq, ws = fp8bq.quant_weight(w32)
            del w32
        g.manual_seed(7)
        a = torch.randn((m, k), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        aq, as_ = fp8bq.quant_act(a)
        c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        def call():
            st = plan.lib.fp8bq_gemm(m, n, k, aq.data_ptr(), as_.data_ptr(), wq.data_ptr(), ws.data_ptr(),
                                     c.data_ptr(), plan.s)
            if st:
                raise fp8bq.Fp8bqError("fp8bq_gemm", st)

        # warm-up window (the first tens of MFMA-bound calls run up to ~20%
        # slower while the clock settles), then three timed windows; the
        # median window is reported
        for _ in range(reps):
            call()
        windows = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(plan.stream)
            for _ in range(reps):
                call()
            e1.record(plan.stream)
            e1.synchronize()
            windows.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = sorted(windows)[1]
        tflops = 2.0 * m * n * k / (us * 1e-6) / 1e12
        out.append({"M": m, "N": n, "K": k, "us": round(us, 2), "us_windows": [round(w, 2) for w in windows],
                    "TFLOPs": round(tflops, 1), "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
                    "scaled_mfma_loop_TFLOPs": round(scaled_loop, 1),
                    "frac_of_scaled_mfma_loop": round(tflops / scaled_loop, 4),
                    "vendor_fp8_gemm_context": vendor_fp8_gemm(m, n, k, reps)})
        del a, aq, as_, c
    return out


def vendor_fp8_gemm(m, n, k, reps):
    """For context only (not this library's path): the same (M, N, K) through
    torch._scaled_mm on e4m3fn tensors with one scale per tensor (the ROCm
    build routes it to hipBLASLt), i.e. an FP8 GEMM without the block scales'
    per-group work, timed like prefill(). None where unsupported."""
    dev = torch.device("cuda:0")
    try:
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        a8 = torch.randn((m, k), generator=g, device=dev).mul_(100.0).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        w8 = torch.randn((n, k), generator=g, device=dev).mul_(100.0).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        one = torch.ones((), device=dev)

        def call():
            return torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)

        for _ in range(reps):
            call()
        windows = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            e1.synchronize()
            windows.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = sorted(windows)[1]
        tflops = 2.0 * m * n * k / (us * 1e-6) / 1e12
        return {"what": "torch._scaled_mm e4m3fn, per-tensor scales (hipBLASLt), no block scales", "us": round(us, 2),
                "TFLOPs": round(tflops, 1), "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4)}
    except (RuntimeError, AttributeError, TypeError) as e:
        return {"what": "torch._scaled_mm unsupported here", "error": str(e)[:200]}


def two_stage(reps=50):
    """Two-stage vocabulary scoring (page 1, "single-stream optimisation"):
    coarse logits from the fused block-FP8 GEMM against the FP8 vocabulary
    projection (V = 152064 stand-in, K = 5120), exact top-64
    (fp8bq_topk_bf16), exact bf16 rescoring of the 64 survivors
    (fp8bq_rescore_bf16). Per M: microseconds of each stage and of the whole
    pipeline (HIP events on the launch stream around `reps` back-to-back
    calls, buffers preallocated), and, for context, torch's bf16 matmul of
    the full projection (the one-stage read the scheme replaces)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    L = fp8bq.lib()
    v, k, kk = workloads.VOCAB, workloads.HIDDEN, workloads.SURVIVORS
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    w32 = torch.randn((v, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
    wq, ws = fp8bq.quant_weight(w32)
    wbf = w32.to(torch.bfloat16)
    del w32
    out = []
    for m in (1, 4, 8, 16):
        g.manual_seed(m)
        h = torch.randn((m, k), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        logits = torch.empty((m, v), dtype=torch.bfloat16, device=dev)
        wsb = fp8bq.topk_workspace_bytes(m, v, kk)
        work = torch.empty(wsb, dtype=torch.uint8, device=dev)
        idx = torch.empty((m, kk), dtype=torch.int32, device=dev)
        val = torch.empty((m, kk), dtype=torch.bfloat16, device=dev)
        scores = torch.empty((m, kk), dtype=torch.float32, device=dev)
        pick = torch.empty((m,), dtype=torch.int32, device=dev)
        hq = torch.empty((m, k), dtype=torch.uint8, device=dev)
        hs = torch.empty((m, k // 128), dtype=torch.float32, device=dev)

        def coarse():
            # the same logits either way (bitwise); the fused launch up to 8
            # tokens, quantisation + GEMM beyond, as fp8bq.two_stage does
            if m <= fp8bq.TWO_STAGE_FUSED_MAX_M:
                st = L.fp8bq_gemm_fused(m, v, k, h.data_ptr(), wq.data_ptr(), ws.data_ptr(), logits.data_ptr(), s)
            else:
                st = L.fp8bq_quant_act(m, k, h.data_ptr(), hq.data_ptr(), hs.data_ptr(), s) or L.fp8bq_gemm(
                    m, v, k, hq.data_ptr(), hs.data_ptr(), wq.data_ptr(), ws.data_ptr(), logits.data_ptr(), s)
            if st:
                raise fp8bq.Fp8bqError("coarse logits", st)

        def select():
            st = L.fp8bq_topk_bf16(m, v, kk, logits.data_ptr(), work.data_ptr(), wsb, idx.data_ptr(),
                                   val.data_ptr(), s)
            if st:
                raise fp8bq.Fp8bqError("fp8bq_topk_bf16", st)

        def exact():
            st = L.fp8bq_rescore_bf16(m, k, v, kk, h.data_ptr(), wbf.data_ptr(), idx.data_ptr(), scores.data_ptr(),
                                      pick.data_ptr(), s)
            if st:
                raise fp8bq.Fp8bqError("fp8bq_rescore_bf16", st)

        def pipeline():
            coarse()
            select()
            exact()

        def full_bf16():
            torch.matmul(h, wbf.t())

        row = {"M": m, "V": v, "K": k, "k": kk}
        for name, fn in (("coarse_us", coarse), ("topk_us", select), ("rescore_us", exact),
                         ("pipeline_us", pipeline), ("torch_bf16_full_us", full_bf16)):
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            e1.synchronize()
            row[name] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
        row["coarse_GBps"] = round(bf16_act_bytes(m, v, k) / (row["coarse_us"] * 1e-6) / 1e9, 1)
        # bytes the pipeline must move: the FP8 projection and its scales, the
        # survivors' bf16 rows, the hidden state, the logits written and read
        pipe_bytes = bf16_act_bytes(m, v, k) + 2 * m * v + 2 * m * kk * k
        row["pipeline_GBps"] = round(pipe_bytes / (row["pipeline_us"] * 1e-6) / 1e9, 1)
        row["bf16_full_bytes"] = 2 * v * k
        out.append(row)
        print(f"bench: two-stage M={m}: {row}", file=sys.stderr, flush=True)
    return out


SWEEP_M = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 33, 48, 49, 64, 65, 80, 81, 96, 128, 129, 192, 256, 384,
           512, 1024, 2048, 3465, 4096]


def m_sweep():
    """fp8bq_gemm over an M grid on the five logged shapes: microseconds per
    call (HIP events on the launch stream, weights rotating over >= 1 GiB of
    copies), GB/s of algorithmic bytes and TFLOP/s; where fp8bq_gemm_ws
    splits K (fp8bq_gemm_workspace_bytes > 0) also its time with the
    workspace. The dispatch boundaries (8/9, 16/17, 32/33, 48/49, 64/65,
    80/81, 128/129) are in the grid on purpose."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s = ctypes.c_void_p(stream.cuda_stream)
    L = fp8bq.lib()
    g = torch.Generator(device=dev)
    rows = []
    mmax = max(SWEEP_M)
    for n, k in workloads.SHAPES:
        copies = max(2, -(-(1 << 30) // (n * k)))
        ws = []
        for i in range(copies):
            g.manual_seed(500 + i)
            w32 = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
            ws.append(fp8bq.quant_weight(w32))
            del w32
        g.manual_seed(77)
        a = torch.randn((mmax, k), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        aq, as_ = fp8bq.quant_act(a)
        c = torch.empty((mmax, n), dtype=torch.bfloat16, device=dev)
        wbytes = {m: L.fp8bq_gemm_workspace_bytes(m, n, k) for m in SWEEP_M}
        work = torch.empty(max(16, max(wbytes.values())), dtype=torch.uint8, device=dev)

        def timed(call, m):
            reps = 8 * copies if m <= 256 else 12
            for i in range(reps):
                call(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                call(i)
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        for m in SWEEP_M:
            def call(i):
                wq, wsc = ws[i % copies]
                st = L.fp8bq_gemm(m, n, k, aq.data_ptr(), as_.data_ptr(), wq.data_ptr(), wsc.data_ptr(), c.data_ptr(), s)
                if st:
                    raise fp8bq.Fp8bqError("fp8bq_gemm", st)

            def call_ws(i):
                wq, wsc = ws[i % copies]
                st = L.fp8bq_gemm_ws(m, n, k, aq.data_ptr(), as_.data_ptr(), wq.data_ptr(), wsc.data_ptr(), c.data_ptr(),
                                     work.data_ptr(), work.numel(), s)
                if st:
                    raise fp8bq.Fp8bqError("fp8bq_gemm_ws", st)
            us = timed(call, m)
            path = L.fp8bq_gemm_path(m, n, k)
            if path == fp8bq.PATH_TILED:
                path = L.fp8bq_gemm_tile_shape(m, n, k)
            row = {"N": n, "K": k, "M": m, "path": fp8bq.PATH_NAMES[path],
                   "us": round(us, 2), "GBps": round(gemm_bytes(m, n, k) / (us * 1e-6) / 1e9, 1),
                   "TFLOPs": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)}
            if wbytes[m] > 0:  # fp8bq_gemm_ws splits K here: its time and number of K parts
                row["ws_us"] = round(timed(call_ws, m), 2)
                row["ws_k_parts"] = wbytes[m] // (4 * m * n)
            rows.append(row)
            print(f"bench: sweep N={n} K={k} M={m}: {us:.2f} us" +
                  (f", with workspace {row['ws_us']:.2f} us" if "ws_us" in row else ""), file=sys.stderr, flush=True)
        del ws, a, aq, as_, c, work
        torch.cuda.empty_cache()
    return rows


READ_GRIDS = (256, 512, 1024, 2048)


# Set by --launch-loop: graph_us times plain launch loops instead of graph
# replays (for profilers that count per kernel dispatch).
LAUNCH_LOOP = False


def loop_us(launch, count):
    """Median over three event-timed windows of `count` back-to-back direct
    launches after one untimed window, microseconds per launch (includes
    the host's launch rate wherever a call is shorter than its launch)."""
    stream = torch.cuda.current_stream()
    for i in range(count):
        launch(i)
    runs = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(count):
            launch(i)
        e1.record(stream)
        e1.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / count)
    return sorted(runs)[1]


def graph_us(launch, count):
    """Median over three replays of a HIP graph of `count` back-to-back
    launches (launch(i) enqueues the i-th), microseconds per launch. Graph
    replays keep the host's launch rate (several microseconds per call
    through Python) out of the figure. With LAUNCH_LOOP set: loop_us."""
    if LAUNCH_LOOP:
        return loop_us(launch, count)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / count)
    del g
    return sorted(runs)[1]


def best_read_us(views, sink):
    """Fastest streaming read (fp8bq_mb_read, twelve 16-byte loads in flight
    per lane) of one buffer of `views` over the grid sizes READ_GRIDS, the
    launches rotating over the views: (us per read, grid)."""
    best = None
    for grid in READ_GRIDS:
        us = graph_us(lambda i: fp8bq.mb_read(views[i % len(views)], grid, sink), max(24, 2 * len(views)))
        if best is None or us < best[0]:
            best = (us, grid)
    return best


def ceilings():
    """What this GPU delivers, to read the roofline fractions against besides
    the published peaks (the library's measurement kernels), each as HIP
    graph replays (graph_us):
    - the streaming-read time of each transfer size the GEMM moves per call
      (the five shapes' bytes at M = 1, the vocabulary projection, 1 GiB):
      the fastest of 256 .. 2048 workgroups of 512 threads, twelve loads in
      flight per lane, buffers rotating over >= 1 GiB;
    - one empty launch of the decode kernels' grid (256 x 512): the fixed
      cost each call pays;
    - the FP8 16x16x128 MFMA rate of 1024 workgroups x 4 waves x 8
      independent chains (the matrix-core peak at the clock this load runs),
      on one code, on quantised Gaussian codes, and with the block-scaled
      GEMM's 4 fp32 scale FMAs per MFMA."""
    dev = torch.device("cuda:0")
    sizes = [(f"({n}, {k}) at M=1", gemm_bytes(1, n, k)) for n, k in workloads.SHAPES]
    sizes += [("vocabulary projection (152064, 5120)", 152064 * 5120), ("1 GiB", 1 << 30)]
    pool = torch.empty(3 << 30, dtype=torch.uint8, device=dev)
    pool.random_(0, 256)
    sink = torch.empty(max(READ_GRIDS), dtype=torch.int32, device=dev)
    read = []
    for name, nbytes in sizes:
        nbytes = nbytes // 256 * 256
        copies = max(2, min(pool.numel() // nbytes, -(-(1 << 30) // nbytes) + 1))
        views = [pool[i * nbytes:(i + 1) * nbytes] for i in range(copies)]
        us, grid = best_read_us(views, sink)
        read.append({"what": name, "bytes": nbytes, "us": round(us, 2), "grid": grid,
                     "GBps": round(nbytes / us / 1e3, 1), "pct_of_8TBps": round(nbytes / us / 1e3 / 80, 1)})
        print(f"bench: read {name} {nbytes} B: {us:.2f} us (grid {grid})", file=sys.stderr, flush=True)
    del pool, views
    torch.cuda.empty_cache()
    empty_us = graph_us(lambda i: fp8bq.mb_empty(256, 512), 500)
    print(f"bench: empty launch {empty_us:.3f} us", file=sys.stderr, flush=True)
    grid, iters = 1024, 4096
    msink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    mfma_us = graph_us(lambda i: fp8bq.mb_mfma(grid, iters, sink=msink), 3)
    flops = grid * 4 * 8 * iters * 2.0 * 16 * 16 * 128
    # the same loop on quantised Gaussian operands (a GEMM's switching
    # activity): the rate the power budget leaves a real FP8 GEMM
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    vals = torch.randn(fp8bq.MB_MFMA_DATA_BYTES, generator=g, device=dev).mul_(448.0 / 4.0)
    codes = vals.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    data_us = graph_us(lambda i: fp8bq.mb_mfma_data(grid, iters, codes, sink=msink), 3)
    # and in the block-scaled GEMM's inner loop (fresh products, 4 fp32
    # scale FMAs per MFMA): the most a per-group-scaled GEMM gets from the
    # matrix cores
    scaled = scaled_mfma_tflops(dev, grid, iters)
    print(f"bench: MFMA loop {flops / mfma_us / 1e6:.0f} TFLOP/s (one code), {flops / data_us / 1e6:.0f} "
          f"(Gaussian codes), {scaled:.0f} (Gaussian codes, 4 scale FMAs per MFMA)", file=sys.stderr, flush=True)
    return {"read": read, "empty_launch_us": round(empty_us, 3),
            "mfma_e4m3_16x16x128": {"TFLOPs": round(flops / mfma_us / 1e6, 1), "us": round(mfma_us, 1),
                                    "frac_of_5000": round(flops / mfma_us / 1e6 / FP8_PEAK_TFLOPS, 4)},
            "mfma_e4m3_16x16x128_gaussian_codes": {
                "TFLOPs": round(flops / data_us / 1e6, 1), "us": round(data_us, 1),
                "frac_of_5000": round(flops / data_us / 1e6 / FP8_PEAK_TFLOPS, 4)},
            "mfma_e4m3_16x16x128_gaussian_codes_scale_fmas": {
                "TFLOPs": round(scaled, 1), "frac_of_5000": round(scaled / FP8_PEAK_TFLOPS, 4)}}


PER_SHAPE_M = [1, 2, 3, 4, 5, 6, 7, 8, 16, 32, 64]


def per_shape(shapes=None):
    """The decode, verify and batch configurations on all five logged shapes
    (or the (N, K) pairs in `shapes`)
    (page 2, section 8): fp8bq_gemm at M = 1..8, 16, 32, 64 and
    fp8bq_gemm_fused at M = 1..8, each as HIP graph replays of
    back-to-back calls with the weights rotating over >= 1 GiB of copies (no
    call finds its weight in the 256 MB Infinity Cache). Per call: us, GB/s
    of algorithmic bytes, % of 8 TB/s, and % of the fastest streaming read of
    the same weight bytes over the same rotating buffers (`read_us`). Per
    shape: the no-cliff ratio max over M = 2..8 of t(M) / t(1)."""
    dev = torch.device("cuda:0")
    L = fp8bq.lib()
    g = torch.Generator(device=dev)
    mmax = max(PER_SHAPE_M)
    sink = torch.empty(max(READ_GRIDS), dtype=torch.int32, device=dev)
    out = []
    for n, k in shapes or workloads.SHAPES:
        copies = max(4, -(-(1 << 30) // (n * k)))
        g.manual_seed(4242)
        w32 = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
        wq0, ws0 = fp8bq.quant_weight(w32)
        del w32
        ws = [(wq0.clone(), ws0.clone()) for _ in range(copies)]  # distinct buffers, same contents
        del wq0, ws0
        a = workloads.activation(mmax, n, k).to(dev)
        aq, as_ = fp8bq.quant_act(a)
        c = torch.empty((mmax, n), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        read_us, read_grid = best_read_us([wq for wq, _ in ws], sink)
        row = {"N": n, "K": k, "weight_copies": copies, "read_us": round(read_us, 2), "read_grid": read_grid,
               "read_pct_of_8TBps": round(100 * n * k / (read_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
               "gemm": [], "fused": []}
        for kind in ("gemm", "fused"):
            for m in PER_SHAPE_M:
                if kind == "fused" and m > 8:
                    continue

                def call(i):
                    wq, wsc = ws[i % copies]
                    s = torch.cuda.current_stream(dev).cuda_stream  # the capturing stream
                    if kind == "gemm":
                        st = L.fp8bq_gemm(m, n, k, aq.data_ptr(), as_.data_ptr(), wq.data_ptr(), wsc.data_ptr(),
                                          c.data_ptr(), s)
                    else:
                        st = L.fp8bq_gemm_fused(m, n, k, a.data_ptr(), wq.data_ptr(), wsc.data_ptr(), c.data_ptr(), s)
                    if st:
                        raise fp8bq.Fp8bqError(f"fp8bq_{kind}", st)

                us = graph_us(call, max(24, 2 * copies))
                nbytes = gemm_bytes(m, n, k) if kind == "gemm" else bf16_act_bytes(m, n, k)
                gbs = nbytes / (us * 1e-6) / 1e9
                row[kind].append({"M": m, "us": round(us, 2), "GBps": round(gbs, 1),
                                  "pct_of_8TBps": round(100 * gbs / HBM_PEAK_GBS, 1),
                                  "pct_of_read": round(100 * read_us / us, 1)})
            t = {r["M"]: r["us"] for r in row[kind]}
            row[f"no_cliff_{kind}"] = round(max(t[m] for m in range(2, 9)) / t[1], 3)
        print(f"bench: per-shape N={n} K={k}: read {read_us:.2f} us, gemm M=1 {row['gemm'][0]['us']} us, "
              f"fused M=1 {row['fused'][0]['us']} us", file=sys.stderr, flush=True)
        out.append(row)
        del ws, a, aq, as_, c
        torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(rows=N, runs=5, runs_one_thread=3):
    """The CPU oracle (numpy, fp64 GEMM) on the workload: activation
    quantisation (quant_act_ref) and the GEMM (gemm_ref) for M = 1..8
    against the first `rows` weight rows of (N, K) = (17408, 5120) (all of
    them by default: about 20 s of CPU work on a 16-thread host), the weight
    pre-quantised. One warm-up pass, then the median of `runs` passes with
    the host's threads (all cores this process may use, at most the
    OMP_NUM_THREADS share when that is set) and of `runs_one_thread` passes
    with one thread. Also the plain fp64 matmul alone on pre-dequantised
    operands (the oracle's arithmetic without its decode and per-group loop).
    Reported in GB/s of the same algorithmic bytes as the GPU figure, and as
    us per call over the full N."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import e4m3_decode, gemm_ref, quant_act_ref, quant_weight_ref

    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    blocks = [quant_weight_ref(workloads.weight_block(N, K, b)) for b in range(rows // 128)]
    w_q = np.concatenate([q for q, _ in blocks])
    w_s = np.concatenate([s for _, s in blocks])
    acts = {m: workloads.activation(m, N, K) for m in MS}
    sample_bytes = sum(bf16_act_bytes(m, rows, K) for m in MS)

    def one_pass():
        t0 = time.perf_counter()
        for m in MS:
            a_q, a_s = quant_act_ref(acts[m])
            gemm_ref(a_q, a_s, w_q, w_s)
        return time.perf_counter() - t0

    def median_pass(count):
        one_pass()
        return float(np.median([one_pass() for _ in range(count)]))

    # the same sums with operands already decoded and scaled, one fp64 matmul per M
    w_deq = e4m3_decode(w_q) * np.repeat(np.repeat(w_s.astype(np.float64), 128, axis=0)[:rows], 128, axis=1)
    a_deq = {}
    for m in MS:
        a_q, a_s = quant_act_ref(acts[m])
        a_deq[m] = e4m3_decode(a_q) * np.repeat(a_s.astype(np.float64), 128, axis=1)

    def matmul_pass():
        t0 = time.perf_counter()
        for m in MS:
            a_deq[m] @ w_deq.T
        return time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        t_all = median_pass(runs)
        matmul_pass()
        t_mm = float(np.median([matmul_pass() for _ in range(runs)]))
    with threadpool_limits(limits=1):
        t_one = median_pass(runs_one_thread)
    scale = N / rows  # calls over the full weight take N / rows times the sample
    return {
        "value": round(sample_bytes / t_all / 1e9, 4),
        "unit": "GB/s",
        "cores": used,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"quant_act_ref + gemm_ref for M=1..8 on " +
                   ("all " if rows == N else f"the first {rows} of ") + f"{N} weight rows (K={K}); median of {runs} "
                   f"passes after 1 warm-up ({runs_one_thread} with one thread)"),
        "pass_s": round(t_all, 4),
        "us_per_call_full_N": round(t_all / len(MS) * scale * 1e6, 1),
        "one_thread": {"value": round(sample_bytes / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                       "pass_s": round(t_one, 4),
                       "us_per_call_full_N": round(t_one / len(MS) * scale * 1e6, 1)},
        "matmul_only": {"what": "fp64 A_deq @ W_deq.T per M, operands pre-dequantised", "pass_s": round(t_mm, 4),
                        "value": round(sample_bytes / t_mm / 1e9, 4), "unit": "GB/s",
                        "us_per_call_full_N": round(t_mm / len(MS) * scale * 1e6, 1)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--kernel-reps", type=int, default=96)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="seconds of the step workload run before any timing (clock and TLB settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=3465 prefill GEMM timing")
    ap.add_argument("--no-two-stage", action="store_true", help="skip the two-stage vocabulary scoring timing")
    ap.add_argument("--no-per-shape", action="store_true",
                    help="skip the all-shapes decode/verify/batch leg (M = 1..8, 16, 32, 64 on the five shapes)")
    ap.add_argument("--only", choices=("prefill", "two-stage", "per-shape", "cpu"),
                    help="run only this leg and print its JSON line (for profiling one kernel family)")
    ap.add_argument("--m-sweep", action="store_true",
                    help="instead of the benchmark, time fp8bq_gemm over an M grid on the five shapes (one JSON line)")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the benchmark, measure the streaming-read, launch and FP8 MFMA ceilings "
                         "(one JSON line)")
    ap.add_argument("--shape", action="append", default=[], metavar="N,K",
                    help="per-shape leg: only this weight shape (repeatable; default: the five logged shapes)")
    ap.add_argument("--launch-loop", action="store_true",
                    help="per-shape leg and ceilings: time event-bracketed launch loops instead of HIP graph "
                         "replays (for rocprofv3 counter runs, which count per dispatch)")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a dispatch of known traffic for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    global LAUNCH_LOOP
    LAUNCH_LOOP = args.launch_loop
    shapes = [tuple(int(x) for x in sh.split(",")) for sh in args.shape] or None
    if shapes and any(sh not in workloads.SHAPES for sh in shapes):
        print(f"--shape must name one of the logged shapes {workloads.SHAPES}", file=sys.stderr)
        sys.exit(2)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    if args.only == "cpu":  # the CPU oracle alone (no GPU needed)
        print(json.dumps({"metric": "CPU oracle", "cpu_baseline": cpu_baseline()}), flush=True)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calibration_copy_mb > 0:
        nbytes = args.calibration_copy_mb << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()

    if args.only == "two-stage":
        print(json.dumps({"metric": "two-stage vocabulary scoring us/call", "data": "synthetic",
                          "two_stage": two_stage(), "device": torch.cuda.get_device_name(0)}), flush=True)
        return
    if args.only == "per-shape":
        print(json.dumps({"metric": "block-FP8 GEMM us/call, five shapes", "data": "synthetic",
                          "per_shape": per_shape(shapes), "device": torch.cuda.get_device_name(0)}), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps({"metric": "prefill block-FP8 GEMM us/call", "data": "synthetic",
                          "prefill": prefill(Plan(1)), "device": torch.cuda.get_device_name(0)}), flush=True)
        return

    if args.ceilings:
        print(json.dumps({"metric": "measured ceilings", "data": "synthetic", **ceilings(),
                          "device": torch.cuda.get_device_name(0)}), flush=True)
        return

    if args.m_sweep:
        print(json.dumps({"metric": "fp8bq_gemm us/call over M", "data": "synthetic", "rows": m_sweep(),
                          "device": torch.cuda.get_device_name(0)}), flush=True)
        return

    w_bytes = N * K
    copies = max(4, -(-(1 << 30) // w_bytes))  # >= 1 GiB of distinct weights
    print(f"bench: preparing {copies} weight copies of N={N} K={K} ({copies * w_bytes / 1e9:.2f} GB)",
          file=sys.stderr, flush=True)
    plan = Plan(copies)

    # Clock and TLB settling before anything is timed: a fixed stretch of
    # the same workload (with only a few warm-up steps the first timed loop
    # read ~5% slow while the clocks ramp and the 13 weight copies' pages are
    # first touched). Then the W warm-up steps and the K timed steps.
    print(f"bench: settling for {args.settle_s} s, then {args.warmup} warm-up and {args.steps} timed steps",
          file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            plan.step_fused()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        plan.step_fused()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(plan.stream)
    for _ in range(args.steps):
        plan.step_fused()
    e1.record(plan.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    def time_steps(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ea = torch.cuda.Event(enable_timing=True)
        eb = torch.cuda.Event(enable_timing=True)
        ea.record(plan.stream)
        for _ in range(args.steps):
            fn()
        eb.record(plan.stream)
        torch.cuda.synchronize()
        return ea.elapsed_time(eb) / args.steps

    # the same workload as two calls per M (quant_act, gemm), and through
    # the weight-only entry point (one launch per M)
    ms_unfused = time_steps(plan.step)
    ms_w8a16 = time_steps(plan.step_w8a16)
    fused_step_bytes = sum(bf16_act_bytes(m, N, K) for m in MS)

    kt = time_kernels(plan, args.kernel_reps)
    unfused_step_bytes = sum(gemm_bytes(m, N, K) + quant_bytes(m, K) for m in MS)
    value = fused_step_bytes / (ms_per_step * 1e-3) / 1e9

    per_m = []
    for m in MS:
        us = kt[("fused", m)]
        gbs = bf16_act_bytes(m, N, K) / (us * 1e-6) / 1e9
        per_m.append({"M": m, "fused_us": round(us, 3), "fused_GBps": round(gbs, 1),
                      "fused_pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                      "gemm_us": round(kt[("gemm", m)], 3),
                      "gemm_GBps": round(gemm_bytes(m, N, K) / (kt[("gemm", m)] * 1e-6) / 1e9, 1),
                      "quant_act_us": round(kt[("quant", m)], 3),
                      "w8a16_us": round(kt[("w8a16", m)], 3),
                      "w8a16_GBps": round(bf16_act_bytes(m, N, K) / (kt[("w8a16", m)] * 1e-6) / 1e9, 1)})
    g_bytes = sum(bf16_act_bytes(m, N, K) for m in MS)
    g_time = sum(kt[("fused", m)] for m in MS) * 1e-6
    achieved = g_bytes / g_time / 1e9
    digest = kernel_source_digest()
    traffic = stored_traffic(digest)

    rec = {
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
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": "decode/verify M=1..8 x (N=17408, K=5120): per-token activation quantisation + block-FP8 "
                        "gemm per M, one fused launch each (fp8bq_gemm_fused)",
            "M": MS, "N": N, "K": K, "weight_copies": copies, "step_bytes": fused_step_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
            "parallelism": "single GPU",
        },
        "per_m": per_m,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "gemm_rows_kernel<16, 8, 5, 5, 6, 2, TOK> (fused quantisation + GEMM; TOK = 1, 2, 4, 8 for "
                      "M = 1, 2, 3..4, 5..8; the M=1..8 launches, HIP events on the launch stream around "
                      "back-to-back launches)",
        },
        "unfused": {
            "path": "fp8bq_quant_act then fp8bq_gemm per M (two launches), same weights and activations",
            "ms_per_step": round(ms_unfused, 5),
            "value": round(unfused_step_bytes / (ms_unfused * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "step_bytes": unfused_step_bytes,
        },
        "w8a16": {
            "path": "fp8bq_gemm_w8a16 (bf16 activation x block-FP8 weight, no activation quantisation), "
                    "one launch per M, same weights and activations",
            "ms_per_step": round(ms_w8a16, 5),
            "value": round(fused_step_bytes / (ms_w8a16 * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "step_bytes": fused_step_bytes,
        },
        "wall_s_timed": round(wall, 3),
        "settle_s": args.settle_s,
        "kernel_source_digest": digest,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_prefill:
        print("bench: timing the prefill GEMMs", file=sys.stderr, flush=True)
        rec["prefill"] = prefill(plan)
    del plan
    torch.cuda.empty_cache()
    if not args.no_per_shape:
        print("bench: timing the five shapes at M = 1..8, 16, 32, 64", file=sys.stderr, flush=True)
        rec["per_shape"] = per_shape()
    if not args.no_two_stage:
        print("bench: timing two-stage vocabulary scoring", file=sys.stderr, flush=True)
        rec["two_stage"] = two_stage()
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
