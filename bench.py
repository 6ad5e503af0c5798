#!/usr/bin/env python3
"""Benchmark of the Tensor Cache hot path on one MI355X.

One step = one fused Tensor Cache layer (sliding-window softmax L1 + L2
outer-product memory read + gate, which includes the eviction-conditioned
writes and the chunked scan) over B=1, H=16, T=32768, d=128, W=1024 with
bf16 inputs and fp32 state.  The other entry points (prefill scan, streaming
decode, delta-rule scan) are timed on their own workloads and reported under
"components".

Prints ONE JSON line.  All inputs are synthetic and resident in HBM before
the timed region; timing uses HIP events on the stream the library launches
on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "memory-scan tokens/s (B·H·T/s) + % of MFMA or HBM roofline, d=128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed calls first: the GPU needs some tens of ms of load to reach its steady clock")
    ap.add_argument("--no-components", action="store_true", help="time only the fused layer")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps to time (default: the workload's 4096; 1024 for the 4x side run); "
                         "short runs are for profiler counter passes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fused", "fused_f32", "scan", "scan_bf16", "scan_backward", "layer_backward", "decode", "decode_x4", "decode_layer", "delta",
                                           "delta_f32", "delta_backward", "hebbian", "capacity"], default=None,
                    help="time a single entry point (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy twice (the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- algorithmic work

def fused_flops(B, H, T, d, W, C=64):
    """L1: 4 d flops per (query, key) pair inside the window; L2 per active
    token: (C+1)(dk+dv) for the intra-chunk part plus 4 dk dv for the state
    read and write."""
    pairs = sum(min(W, t + 1) for t in range(min(T, W))) + max(T - W, 0) * W
    l1 = 4 * d * pairs
    l2 = max(T - W, 0) * ((C + 1) * 2 * d + 4 * d * d)
    return B * H * (l1 + l2)


def fused_main_flops(B, H, T, d, W, C=64):
    """Algorithmic work of the fused layer's main kernel: the L1 window
    softmax (4 d per pair) plus the L2 read per active token, (C+1)(dk+dv)
    intra-chunk and 2 dk dv for q.S; the state writes (2 dk dv per eviction)
    belong to the pre-pass."""
    pairs = sum(min(W, t + 1) for t in range(min(T, W))) + max(T - W, 0) * W
    return B * H * (4 * d * pairs + max(T - W, 0) * ((C + 1) * 2 * d + 2 * d * d))


def fused_bytes(B, H, T, d):
    return B * H * T * (3 * d * 2 + d * 4)  # q, k, v bf16 in, y fp32 out


def scan_flops(B, H, T, d, W, C=64):
    return B * H * max(T - W, 0) * ((C + 1) * 2 * d + 4 * d * d)


def scan_bytes(B, H, T, d, in_bytes):
    return B * H * T * (3 * d * in_bytes + d * 4)


def scan_backward_flops(B, H, T, d, W, C=64):
    # three reads of the forward's shape (dq, dk, dv) plus the dlam pass: per
    # active row two in-chunk Gram rows (2 x 2Cd) and four d x d products
    # (two entering-state terms, two state updates)
    return 3 * scan_flops(B, H, T, d, W, C) + B * H * max(T - W, 0) * (4 * C * d + 8 * d * d)


def scan_backward_bytes(B, H, T, d):
    # read q, k, v, dm and write dq, dk, dv once, fp32
    return B * H * T * d * 4 * 7


def window_backward_flops(B, H, T, d, W):
    """Window softmax backward: per (query, key) pair of the window the scores
    (2d), dp = <dy, v> (2d), dv += p dy (2d), dq += ds k (2d) and
    dk += ds q (2d)."""
    pairs = sum(min(W, t + 1) for t in range(min(T, W))) + max(T - W, 0) * W
    return B * H * 10 * d * pairs


def decode_bytes_per_head(d, in_bytes=2):
    # A read + written (fp32), q, k, v in, evicted pair read, new pair written, m out
    return 2 * d * d * 4 + 3 * d * in_bytes + 2 * d * in_bytes + 2 * d * in_bytes + d * 4


def decode_layer_bytes_per_head(d, W, in_bytes=2):
    # the L2 step, plus the other W - 1 ring slots (k and v) read for the window softmax
    return decode_bytes_per_head(d, in_bytes) + 2 * (W - 1) * d * in_bytes


def delta_bytes(B, H, T, d, in_bytes=2):
    return B * H * T * (3 * d * in_bytes + 4 + d * 4)


def delta_flops(B, H, T, d):
    return B * H * T * 6 * d * d  # prediction, write, read per token


def delta_backward_bytes(B, H, T, d, in_bytes=4):
    # read q, k, v (input dtype), do, beta and write dq, dk, dv, dbeta once (fp32)
    return B * H * T * (3 * d * in_bytes + 4 * d * 4 + 8)


def delta_backward_flops(B, H, T, d):
    # the reverse of the per-token rule: per token the forward's prediction,
    # write and read (6 d^2) and their adjoints (12 d^2)
    return B * H * T * 18 * d * d


# ----------------------------------------------------------------------------- timing

def time_calls(fn, steps, warmup, kernel_timer=None):
    """Whole-call time per step (events bracketing the K steps) and, when a
    KernelTimer is given, the mean duration of the main kernel of each call."""
    import torch

    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i, (a, b) in enumerate(ev):
        if kernel_timer is not None:
            kernel_timer.arm(i)
        a.record()
        fn(i)
        b.record()
    t_end.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    total = t_start.elapsed_time(t_end)
    kernel_ms = kernel_timer.mean_ms() if kernel_timer is not None else None
    return total / steps, sum(per) / len(per), kernel_ms


def graph_ms_per_step(launch, n, reps=3):
    """Mean time per step of n consecutive steps captured in one HIP graph
    (torch.cuda.CUDAGraph) and replayed reps times, after one untimed replay:
    the launch gaps between steps shrink to the graph's.  launch(i, stream)
    issues step i on the given stream."""
    import torch

    from linear_attention_tensor_amd import ops

    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st = ops._stream()  # the capturing stream
        for i in range(n):
            launch(i, st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * n)


class KernelTimer:
    """HIP events recorded by the library around an entry point's main kernel
    (tc_profile_next_call), on the stream that kernel is launched on."""

    def __init__(self, n):
        import ctypes

        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.ev.append((a, b))

    def arm(self, i):
        from linear_attention_tensor_amd import _lib

        a, b = self.ev[i]
        _lib.check("tc_profile_next_call", _lib.lib().tc_profile_next_call(a, b))

    def mean_ms(self):
        import ctypes

        out = []
        for a, b in self.ev:
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        for a, b in self.ev:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        return sum(out) / len(out)


def source_files(source):
    """csrc/<source> and the local headers it includes (quoted #include, followed
    recursively), each once, in first-seen order."""
    import re

    csrc = os.path.join(ROOT, "linear_attention_tensor_amd", "csrc")
    seen, todo = [], [source]
    while todo:
        name = todo.pop(0)
        path = os.path.join(csrc, name)
        if name in seen or not os.path.exists(path):
            continue
        seen.append(name)
        todo += re.findall(r'^#include "([^"]+)"', open(path).read(), flags=re.M)
    return seen


def source_digest(source):
    """First 16 hex digits of the SHA-256 of csrc/<source> and its local headers
    (source_files), concatenated: the code a counter summary was taken from."""
    import hashlib

    csrc = os.path.join(ROOT, "linear_attention_tensor_amd", "csrc")
    h = hashlib.sha256()
    for name in source_files(source):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def counters_from_profile(name, source):
    """Fields of a committed rocprofv3 counter summary profiles/<name>.txt
    ("key: value" lines), or None when there is none or its recorded source
    digest no longer matches csrc/<source> and its headers."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path) or not source_files(source):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("source_sha256_16") != source_digest(source):
        return None
    return fields


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic_<kernel>_fused_layer_bf16.txt), or None when
    there is none or the kernel source has changed since."""
    fields = counters_from_profile(f"traffic_{kernel}_fused_layer_bf16", "tc_swa.hip")
    if fields is None or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5), "traffic": traffic}


def to_dev_bf16(arr, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)


def to_dev_f32(arr, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


# ----------------------------------------------------------------------------- workloads

def bench_fused(steps, warmup, dev):
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["fused_layer_bf16"]
    x = I.draw_workload("fused_layer_bf16")
    q, k, v = (to_dev_bf16(x[n], dev) for n in ("q", "k", "v"))
    lam, eta, g = (to_dev_f32(x[n], dev) for n in ("lam", "eta", "g"))
    y = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    A = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(ops.fused_workspace(w.B, w.H, w.T, w.d, w.d, w.W, 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    st = ops._stream()
    scale = 1.0 / math.sqrt(w.d)
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 1, ops._ptr(lam), ops._ptr(eta), ops._ptr(g),
            w.B, w.H, w.T, w.d, w.d, w.W, 64, scale, ops._ptr(y), ops._ptr(A), ops._ptr(ws), ws.numel(), st)

    def call(_):
        s = lib.tc_fused_layer(*args)
        if s != 0:
            raise RuntimeError(ops._lib.last_error())

    kt = KernelTimer(steps)
    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, kt)
    # the same inputs through the L1 cache alone (pure sliding-window softmax)
    y1 = torch.empty_like(y)
    wargs = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 1, w.B, w.H, w.T, w.d, w.d, w.W, scale, ops._ptr(y1), st)

    def call_window(_):
        if lib.tc_window_attention(*wargs) != 0:
            raise RuntimeError(ops._lib.last_error())

    _, ms_window, _ = time_calls(call_window, steps, warmup)
    ms_layer_again, _, _ = time_calls(call, steps, warmup)  # interleaved, against clock drift
    tokens = w.B * w.H * w.T
    flops = fused_flops(w.B, w.H, w.T, w.d, w.W)
    main_flops = fused_main_flops(w.B, w.H, w.T, w.d, w.W)
    res = {
        "workload": w.name, "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
        "roofline": dict(roofline("mfma", main_flops / (kernel_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s",
                                  traffic_from_profile("swa_kernel")),
                         scope="swa_kernel<128> alone: its algorithmic flops / its own event-timed duration"),
        "layer_roofline": dict(roofline("mfma", flops / (ms_call * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
                               scope="whole layer: all algorithmic flops / whole-call time"),
        "main_kernel": {"name": "swa_kernel<128>", "ms": kernel_ms, "algorithmic_flops": main_flops},
        "layer": {"ms_per_call": ms_call, "algorithmic_flops": flops,
                  "tflops": flops / (ms_call * 1e-3) / 1e12,
                  "algorithmic_bytes": fused_bytes(w.B, w.H, w.T, w.d)},
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "chunk": 64,
                   "dtype_in": "bf16",
                   "state": "fp32 (each 256-token tile's contribution passes through bf16 between kernels)"},
    }
    layer_ms = 0.5 * (ms_call + ms_layer_again)
    kv_full = w.T * 2 * w.d                 # a full KV cache per head at this length (elements)
    kv_tc = w.W * 2 * w.d + w.d * w.d       # ring + L2 matrix per head
    res["l2_overhead"] = {
        "layer_ms": layer_ms, "window_only_ms": ms_window,
        "overhead_pct": 100.0 * (layer_ms / ms_window - 1.0),
        "note": "the fused layer (window softmax + L2 write/read + gate) against tc_window_attention (the "
                "window softmax alone) on the same inputs, HIP events, same process",
        "retained_state_ratio_full_kv_over_tc": kv_full / kv_tc,
        "pages_context": "the pages report about 30% throughput overhead over a pure sliding window and 2.4x "
                         "lower peak GPU memory than a full KV cache at L = 32,768, for a whole model, hardware "
                         "not named; context only, not comparable with a kernel timing",
    }
    return res, x


def window_flops(B, H, T, d, W):
    """The window softmax alone: 4 d flops per (query, key) pair inside the window."""
    pairs = sum(min(W, t + 1) for t in range(min(T, W))) + max(T - W, 0) * W
    return B * H * 4 * d * pairs


def bench_fused_f32(steps, warmup, dev, x=None):
    """The fused layer with fp32 inputs at the headline shape (the bf16
    workload's values, held in fp32): the four-piece fp32 prefill scan, then
    the fp32-MFMA window softmax with the gate; and the window alone."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["fused_layer_bf16"]
    if x is None:
        x = I.draw_workload("fused_layer_bf16")
    q, k, v = (to_dev_f32(x[n + "64"], dev) for n in ("q", "k", "v"))
    lam, eta, g = (to_dev_f32(x[n], dev) for n in ("lam", "eta", "g"))
    y = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ops.fused_workspace(w.B, w.H, w.T, w.d, w.d, w.W, 0), 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    st = ops._stream()
    scale = 1.0 / math.sqrt(w.d)
    largs = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, ops._ptr(lam), ops._ptr(eta), ops._ptr(g),
             w.B, w.H, w.T, w.d, w.d, w.W, 64, scale, ops._ptr(y), None, ops._ptr(ws), ws.numel(), st)
    wargs = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, w.B, w.H, w.T, w.d, w.d, w.W, scale, ops._ptr(y), st)

    def call_layer(_):
        if lib.tc_fused_layer(*largs) != 0:
            raise RuntimeError(ops._lib.last_error())

    def call_window(_):
        if lib.tc_window_attention(*wargs) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, _ = time_calls(call_layer, steps, warmup)
    _, ms_window, kernel_ms = time_calls(call_window, steps, warmup, KernelTimer(steps))
    wf = window_flops(w.B, w.H, w.T, w.d, w.W)
    flops = fused_flops(w.B, w.H, w.T, w.d, w.W)
    return {"workload": "fused_layer_f32", "ms_per_step": ms, "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "ms_per_call": ms_call,
            "roofline": dict(roofline("mfma", wf / (kernel_ms * 1e-3) / 1e12, PEAK_FP32_TFLOPS, "TFLOP/s"),
                             scope="window_kernel<float, 128> alone (tc_window_attention, fp32): its algorithmic "
                                   "flops / its own event-timed duration"),
            "layer_tflops": flops / (ms_call * 1e-3) / 1e12,
            "main_kernel": {"name": "window_kernel<float, 128>", "ms": kernel_ms, "algorithmic_flops": wf},
            "window_only_ms_per_call": ms_window,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "f32"}}


def bench_scan(steps, warmup, dev):
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["prefill_scan_f32"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_f32(x[n], dev) for n in ("q", "k", "v"))
    lam, eta = to_dev_f32(x["lam"], dev), to_dev_f32(x["eta"], dev)
    m = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    A = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    nb = ops.scan_workspace(w.B, w.H, w.T, w.d, w.d, w.W, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, ops._ptr(lam), ops._ptr(eta), w.B, w.H, w.T, w.d,
            w.d, w.W, 64, ops._ptr(m), ops._ptr(A), ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.tc_scan_forward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    flops = scan_flops(w.B, w.H, w.T, w.d, w.W)
    nbytes = scan_bytes(w.B, w.H, w.T, w.d, 4)
    tf = flops / (ms_call * 1e-3) / 1e12
    gbs = nbytes / (ms_call * 1e-3) / 1e9
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("mfma", tf, PEAK_FP32_TFLOPS, "TFLOP/s"),
            "hbm": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
            "main_kernel": {"name": "scan_state_fast8 + scan_output_fast8 (the call's two launches)",
                            "ms": kernel_ms}, "ms_per_call": ms_call,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "f32"}}


def bench_scan_bf16(steps, warmup, dev):
    """tc_scan_forward (the L2 read alone) with bf16 inputs at the fused-layer size."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["fused_layer_bf16"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_bf16(x[n], dev) for n in ("q", "k", "v"))
    lam, eta = to_dev_f32(x["lam"], dev), to_dev_f32(x["eta"], dev)
    m = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    A = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    nb = ops.scan_workspace(w.B, w.H, w.T, w.d, w.d, w.W, 1)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 1, ops._ptr(lam), ops._ptr(eta), w.B, w.H, w.T, w.d,
            w.d, w.W, 64, ops._ptr(m), ops._ptr(A), ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.tc_scan_forward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    nbytes = scan_bytes(w.B, w.H, w.T, w.d, 2)
    return {"workload": w.name + " (L2 read only)", "ms_per_step": ms,
            "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("hbm", nbytes / (ms_call * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
            "mfma": roofline("mfma", scan_flops(w.B, w.H, w.T, w.d, w.W, 256) / (ms_call * 1e-3) / 1e12,
                             PEAK_BF16_TFLOPS, "TFLOP/s"),
            "main_kernel": {"name": "scan_read_kernel<128>", "ms": kernel_ms}, "ms_per_call": ms_call,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "bf16"}}


def bench_scan_backward(steps, warmup, dev):
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["prefill_scan_f32"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_f32(x[n], dev) for n in ("q", "k", "v"))
    lam, eta = to_dev_f32(x["lam"], dev), to_dev_f32(x["eta"], dev)
    dm = to_dev_f32(I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed), dev)
    shape = (w.B, w.H, w.T, w.d)
    gq, gk, gv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    glam, geta = (torch.empty((w.H,), dtype=torch.float32, device=dev) for _ in range(2))
    nb = ops.scan_backward_workspace(w.B, w.H, w.T, w.d, w.d, w.W, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    lib = ops.lib()
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, ops._ptr(lam), ops._ptr(eta), None, w.B, w.H, w.T,
            w.d, w.d, w.W, 64, ops._ptr(dm), ops._ptr(gq), ops._ptr(gk), ops._ptr(gv), ops._ptr(glam),
            ops._ptr(geta), None, ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.tc_scan_backward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    flops = scan_backward_flops(w.B, w.H, w.T, w.d, w.W)
    nbytes = scan_backward_bytes(w.B, w.H, w.T, w.d)
    return {"workload": w.name + " backward", "ms_per_step": ms,
            "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("mfma", flops / (ms_call * 1e-3) / 1e12, PEAK_FP32_TFLOPS, "TFLOP/s"),
            "hbm": roofline("hbm", nbytes / (ms_call * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
            "main_kernel": {"name": "scan_bwd_fwd_fast<64>", "ms": kernel_ms},
            "ms_per_call": ms_call,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "f32"}}


def bench_layer_backward(steps, warmup, dev, x=None):
    """tc_fused_layer_backward at the fused layer's size (bf16 inputs, d =
    128): the gated L2-read backward (four d = 64 pieces, fp32) and the window
    softmax backward (bf16 MFMA)."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["fused_layer_bf16"]
    if x is None:
        x = I.draw_workload(w.name)
    q, k, v = (to_dev_bf16(x[n], dev) for n in ("q", "k", "v"))
    lam, eta, g = (to_dev_f32(x[n], dev) for n in ("lam", "eta", "g"))
    dy = to_dev_f32(I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed), dev)
    shape = (w.B, w.H, w.T, w.d)
    gq, gk, gv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    glam, geta, gg = (torch.empty((w.H,), dtype=torch.float32, device=dev) for _ in range(3))
    lib = ops.lib()
    nb = lib.tc_fused_layer_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, w.W, 64, 1)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 1, ops._ptr(lam), ops._ptr(eta), ops._ptr(g), w.B, w.H, w.T,
            w.d, w.d, w.W, 64, 1.0 / math.sqrt(w.d), ops._ptr(dy), ops._ptr(gq), ops._ptr(gk), ops._ptr(gv),
            ops._ptr(glam), ops._ptr(geta), ops._ptr(gg), ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.tc_fused_layer_backward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    # about 10 ms per call: a few untimed calls settle the clock
    ms, ms_call, _ = time_calls(call, max(1, steps // 4), min(warmup, 5))
    wflops = window_backward_flops(w.B, w.H, w.T, w.d, w.W)
    sflops = scan_backward_flops(w.B, w.H, w.T, w.d, w.W)
    flops = wflops + sflops
    # The two parts run on different matrix units: the peak of the call is the
    # rate at which its flop mix would run with each part at its own peak.
    peak = flops / (wflops / PEAK_BF16_TFLOPS + sflops / PEAK_FP32_TFLOPS)
    return {"workload": w.name + " backward", "ms_per_step": ms,
            "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("mfma", flops / (ms_call * 1e-3) / 1e12, round(peak, 3), "TFLOP/s"),
            "roofline_scope": "whole call: the window-softmax backward (bf16 MFMA) plus the gated L2-read "
                              "backward (fp32 MFMA, four d = 64 pieces); peak = the flop mix at the bf16 "
                              "and fp32 MFMA peaks",
            "flops": {"window_backward_bf16": wflops, "l2_read_backward_fp32": sflops},
            "ms_per_call": ms_call, "workspace_bytes": nb,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "bf16"}}


def bench_layer_backward_f32(steps, warmup, dev):
    """tc_fused_layer_backward with fp32 inputs at the batched prefill
    workload (B=4, H=8, T=4096, d=64, W=512): the gated L2-read backward and
    the window softmax backward, both on fp32 MFMA; and the window softmax
    backward alone (tc_window_attention_backward), whose dk/dv kernel the
    library's timing events bracket."""
    import numpy as np
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["prefill_scan_f32"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_f32(x[n], dev) for n in ("q", "k", "v"))
    lam, eta = to_dev_f32(x["lam"], dev), to_dev_f32(x["eta"], dev)
    g = to_dev_f32(np.random.default_rng(3).standard_normal(w.H), dev)
    dy = to_dev_f32(I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed), dev)
    shape = (w.B, w.H, w.T, w.d)
    gq, gk, gv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    glam, geta, gg = (torch.empty((w.H,), dtype=torch.float32, device=dev) for _ in range(3))
    lib = ops.lib()
    scale = 1.0 / math.sqrt(w.d)
    nb = lib.tc_fused_layer_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, w.W, 64, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    largs = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, ops._ptr(lam), ops._ptr(eta), ops._ptr(g), w.B, w.H, w.T,
             w.d, w.d, w.W, 64, scale, ops._ptr(dy), ops._ptr(gq), ops._ptr(gk), ops._ptr(gv),
             ops._ptr(glam), ops._ptr(geta), ops._ptr(gg), ops._ptr(ws), ws.numel(), ops._stream())
    nbw = lib.tc_window_attention_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, w.W, 0)
    wws = torch.empty(max(nbw, 1), dtype=torch.uint8, device=dev)
    wargs = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, w.B, w.H, w.T, w.d, w.d, w.W, scale, ops._ptr(dy),
             ops._ptr(gq), ops._ptr(gk), ops._ptr(gv), ops._ptr(wws), wws.numel(), ops._stream())

    def call_layer(_):
        if lib.tc_fused_layer_backward(*largs) != 0:
            raise RuntimeError(ops._lib.last_error())

    def call_window(_):
        if lib.tc_window_attention_backward(*wargs) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, _ = time_calls(call_layer, steps, warmup)
    _, ms_window, kernel_ms = time_calls(call_window, steps, warmup, KernelTimer(steps))
    wflops = window_backward_flops(w.B, w.H, w.T, w.d, w.W)
    flops = wflops + scan_backward_flops(w.B, w.H, w.T, w.d, w.W)
    return {"workload": w.name + " fused layer backward", "ms_per_step": ms,
            "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3), "ms_per_call": ms_call,
            "roofline": roofline("mfma", flops / (ms_call * 1e-3) / 1e12, PEAK_FP32_TFLOPS, "TFLOP/s"),
            "roofline_scope": "whole call: the window-softmax backward plus the gated L2-read backward, all on "
                              "fp32 MFMA, their algorithmic flops over the fp32 peak",
            "window_backward": {"ms_per_call": ms_window, "kv_kernel_ms": kernel_ms,
                                "tflops": wflops / (ms_window * 1e-3) / 1e12},
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "W": w.W, "dtype_in": "f32"}}


def bench_decode(steps, warmup, dev, n_steps=4096, B=None):
    """The decode workload's L2 step (4096 steps, 64 x 32 heads).  With B
    given (the side run: 256 sequences, 512 MiB of A) the state no longer
    fits the 256 MB Infinity Cache, so every step streams A from HBM."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["decode_bf16"]
    B = w.B if B is None else B
    H, d, W = w.H, w.d, w.W
    gen = torch.Generator(device=dev).manual_seed(w.seed)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    n_steps = min(n_steps, w.steps)
    scale = 1.0 / math.sqrt(d)
    qs = (torch.randn((n_steps, B, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    ks = unit(torch.randn((n_steps, B, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    vs = (torch.randn((n_steps, B, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    ring_k = unit(torch.randn((B, H, W, d), generator=gen, device=dev)).to(torch.bfloat16)
    ring_v = (torch.randn((B, H, W, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    A = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
    sc = I.decode_scalars(H)
    lam, eta = to_dev_f32(sc["lam"], dev), to_dev_f32(sc["eta"], dev)
    pos = (W + torch.arange(n_steps + warmup, device=dev, dtype=torch.int64))[:, None].repeat(1, B).contiguous()
    m = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    lib = ops.lib()
    st = ops._stream()
    P = ops._ptr
    qp = [P(qs[i]) for i in range(n_steps)]
    kp = [P(ks[i]) for i in range(n_steps)]
    vp = [P(vs[i]) for i in range(n_steps)]
    pp = [P(pos[i]) for i in range(n_steps + warmup)]
    rk, rv, Ap, lp, ep, mp = P(ring_k), P(ring_v), P(A), P(lam), P(eta), P(m)
    counter = {"i": 0}

    def call(i):
        j = counter["i"]
        counter["i"] += 1
        s = lib.tc_decode_step(qp[j % n_steps], kp[j % n_steps], vp[j % n_steps], 1, rk, rv, Ap, lp, ep,
                               pp[j], B, H, d, d, W, mp, st)
        if s != 0:
            raise RuntimeError(ops._lib.last_error())

    # warmup steps advance the stream position too; the timed steps continue from there
    ms, ms_call, kernel_ms = time_calls(call, n_steps, warmup, KernelTimer(n_steps))
    # the same steps as one HIP graph (positions continue after the eager ones;
    # every replay repeats them, each step still evicting and writing one slot)
    posg = (W + n_steps + warmup + torch.arange(n_steps, device=dev, dtype=torch.int64))[:, None].repeat(1, B)
    posg = posg.contiguous()
    pg = [P(posg[i]) for i in range(n_steps)]

    def launch(i, stream):
        s = lib.tc_decode_step(qp[i], kp[i], vp[i], 1, rk, rv, Ap, lp, ep, pg[i], B, H, d, d, W, mp, stream)
        if s != 0:
            raise RuntimeError(ops._lib.last_error())

    ms_graph = graph_ms_per_step(launch, n_steps)
    per_head = decode_bytes_per_head(d)
    gbs = B * H * per_head / (kernel_ms * 1e-3) / 1e9
    a_mib = B * H * d * d * 4 / 2 ** 20
    name = w.name if B == w.B else f"{w.name} x{B // w.B} sequences"
    tag = "decode_bf16" if B == w.B else f"decode_bf16_x{B // w.B}"
    res = {"workload": name, "ms_per_step": ms_graph, "tokens_per_s": B * H / (ms_graph * 1e-3),
           "ms_per_step_eager": ms, "tokens_per_s_eager": B * H / (ms * 1e-3),
           "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
           "note": f"ms_per_step: the {n_steps} steps replayed as one HIP graph; eager: one launch per step with "
                   f"per-step events. A is {a_mib:.0f} MiB ({'inside' if a_mib < 256 else 'beyond'} the "
                   f"256 MB Infinity Cache); GB/s is algorithmic bytes / kernel time",
           "main_kernel": {"name": "decode_kernel", "ms": kernel_ms}, "ms_per_call": ms_call,
           "algorithmic_bytes_per_step": B * H * per_head,
           "config": {"B": B, "H": H, "d": d, "W": W, "steps": n_steps, "dtype_in": "bf16"}}
    c = counters_from_profile(f"traffic_decode_kernel_{tag}", "tc_decode.hip")
    if c is not None and "hbm_bytes_per_launch" in c:
        hb = float(c["hbm_bytes_per_launch"])
        res["hbm_counters"] = {"bytes_per_step": hb, "vs_algorithmic": hb / (B * H * per_head),
                               "gbs": hb / (kernel_ms * 1e-3) / 1e9,
                               "frac": hb / (kernel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return res


def bench_decode_layer(steps, warmup, dev, n_steps=256):
    """Full decode step of the layer (ring softmax + L2 + gate) on the decode workload."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["decode_bf16"]
    B, H, d, W = w.B, w.H, w.d, w.W
    gen = torch.Generator(device=dev).manual_seed(w.seed + 1)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    scale = 1.0 / math.sqrt(d)
    qs = (torch.randn((n_steps, B, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    ks = unit(torch.randn((n_steps, B, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    vs = (torch.randn((n_steps, B, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    ring_k = unit(torch.randn((B, H, W, d), generator=gen, device=dev)).to(torch.bfloat16)
    ring_v = (torch.randn((B, H, W, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    A = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
    sc = I.decode_scalars(H)
    lam, eta = to_dev_f32(sc["lam"], dev), to_dev_f32(sc["eta"], dev)
    g = torch.randn((H,), generator=gen, device=dev)
    pos = (W + torch.arange(n_steps + warmup, device=dev, dtype=torch.int64))[:, None].repeat(1, B).contiguous()
    y = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    lib = ops.lib()
    st = ops._stream()
    P = ops._ptr
    qp = [P(qs[i]) for i in range(n_steps)]
    kp = [P(ks[i]) for i in range(n_steps)]
    vp = [P(vs[i]) for i in range(n_steps)]
    pp = [P(pos[i]) for i in range(n_steps + warmup)]
    rk, rv, Ap, lp, ep, gp, yp = P(ring_k), P(ring_v), P(A), P(lam), P(eta), P(g), P(y)
    counter = {"i": 0}

    def call(i):
        j = counter["i"]
        counter["i"] += 1
        s = lib.tc_decode_layer_step(qp[j % n_steps], kp[j % n_steps], vp[j % n_steps], 1, rk, rv, Ap, lp,
                                     ep, gp, pp[j], B, H, d, d, W, scale, yp, st)
        if s != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, n_steps, warmup, KernelTimer(n_steps))
    posg = (W + n_steps + warmup + torch.arange(n_steps, device=dev, dtype=torch.int64))[:, None].repeat(1, B)
    posg = posg.contiguous()
    pg = [P(posg[i]) for i in range(n_steps)]

    def launch(i, stream):
        s = lib.tc_decode_layer_step(qp[i], kp[i], vp[i], 1, rk, rv, Ap, lp, ep, gp, pg[i], B, H, d, d, W,
                                     scale, yp, stream)
        if s != 0:
            raise RuntimeError(ops._lib.last_error())

    ms_graph = graph_ms_per_step(launch, n_steps)
    per_head = decode_layer_bytes_per_head(d, W)
    gbs = B * H * per_head / (kernel_ms * 1e-3) / 1e9
    return {"workload": w.name + " (full layer step)", "ms_per_step": ms_graph,
            "tokens_per_s": B * H / (ms_graph * 1e-3),
            "ms_per_step_eager": ms, "tokens_per_s_eager": B * H / (ms * 1e-3),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
            "note": "ms_per_step: the steps replayed as one HIP graph; eager: one launch per step with per-step "
                    "events. Per head-step: the ring (2 (W-1) d bf16) plus the L2 step; GB/s is algorithmic "
                    "bytes / kernel time",
            "main_kernel": {"name": "decode_layer_kernel", "ms": kernel_ms}, "ms_per_call": ms_call,
            "config": {"B": B, "H": H, "d": d, "W": W, "steps": n_steps, "dtype_in": "bf16"}}


def bench_delta(steps, warmup, dev):
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["delta_scan_bf16"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_bf16(x[n], dev) for n in ("q", "k", "v"))
    beta = to_dev_f32(x["beta"], dev)
    o = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    nb = ops.delta_workspace(w.B, w.H, w.T, w.d, w.d, 1)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 1, ops._ptr(beta), w.B, w.H, w.T, w.d, w.d, 64, None,
            ops._ptr(o), ops._ptr(S), ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.delta_scan_forward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    nbytes = delta_bytes(w.B, w.H, w.T, w.d)
    gbs = nbytes / (ms_call * 1e-3) / 1e9
    tf = delta_flops(w.B, w.H, w.T, w.d) / (ms_call * 1e-3) / 1e12
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
            "mfma": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s"),
            "main_kernel": {"name": "delta_main_kernel<128>", "ms": kernel_ms}, "ms_per_call": ms_call,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "dtype_in": "bf16"}}


def bench_delta_f32(steps, warmup, dev):
    """delta_scan_forward with float32 inputs at the backward's workload."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS["delta_backward_f32"]
    x = I.draw_workload(w.name)
    q, k, v = (to_dev_f32(x[n], dev) for n in ("q", "k", "v"))
    beta = to_dev_f32(x["beta"], dev)
    o = torch.empty((w.B, w.H, w.T, w.d), dtype=torch.float32, device=dev)
    nb = ops.delta_workspace(w.B, w.H, w.T, w.d, w.d, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    lib = ops.lib()
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), 0, ops._ptr(beta), w.B, w.H, w.T, w.d, w.d, 64, None,
            ops._ptr(o), None, ops._ptr(ws), ws.numel(), ops._stream())

    def call(_):
        if lib.delta_scan_forward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    gbs = delta_bytes(w.B, w.H, w.T, w.d, 4) / (ms_call * 1e-3) / 1e9
    return {"workload": "delta_scan_f32", "ms_per_step": ms, "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
            "main_kernel": {"name": "delta_fwd_walk<64>", "ms": kernel_ms}, "ms_per_call": ms_call,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "dtype_in": "f32"}}


def bench_delta_backward(steps, warmup, dev, workload="delta_backward_f32", bf16=False):
    """delta_scan_backward: fp32 inputs at d = 64, or the delta-rule workload
    itself (bf16 inputs, d = 128; the state rows in pieces of 16)."""
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.WORKLOADS[workload]
    x = I.draw_workload(w.name)
    conv = to_dev_bf16 if bf16 else to_dev_f32
    q, k, v = (conv(x[n], dev) for n in ("q", "k", "v"))
    beta = to_dev_f32(x["beta"], dev)
    do = to_dev_f32(I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed), dev)
    shape = (w.B, w.H, w.T, w.d)
    gq, gk, gv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    gb = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    lib = ops.lib()
    dt = 1 if bf16 else 0
    nb = lib.delta_scan_backward_workspace_bytes(w.B, w.H, w.T, w.d, w.d, 64, dt)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    args = (ops._ptr(q), ops._ptr(k), ops._ptr(v), dt, ops._ptr(beta), w.B, w.H, w.T, w.d, w.d, 64, None,
            ops._ptr(do), None, ops._ptr(gq), ops._ptr(gk), ops._ptr(gv), ops._ptr(gb), None, ops._ptr(ws),
            ws.numel(), ops._stream())

    def call(_):
        if lib.delta_scan_backward(*args) != 0:
            raise RuntimeError(ops._lib.last_error())

    ms, ms_call, kernel_ms = time_calls(call, steps, warmup, KernelTimer(steps))
    gbs = delta_backward_bytes(w.B, w.H, w.T, w.d, 2 if bf16 else 4) / (ms_call * 1e-3) / 1e9
    tf = delta_backward_flops(w.B, w.H, w.T, w.d) / (ms_call * 1e-3) / 1e12
    kernel = "delta_bwd_grads_pieces" if w.d == 128 else f"delta_bwd_grads<{w.d}>"
    return {"workload": f"{w.name} backward" if bf16 else w.name, "ms_per_step": ms,
            "tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s"),
            "mfma": roofline("mfma", tf, PEAK_FP32_TFLOPS, "TFLOP/s"),
            "main_kernel": {"name": kernel, "ms": kernel_ms}, "ms_per_call": ms_call,
            "workspace_bytes": nb,
            "config": {"B": w.B, "H": w.H, "T": w.T, "d": w.d, "dtype_in": "bf16" if bf16 else "f32"}}


def bench_hebbian(steps, warmup, dev):
    import numpy as np
    import torch

    from linear_attention_tensor_amd import inputs as I
    from linear_attention_tensor_amd import ops

    w = I.FACT_WORKLOADS["hebbian_f32"]
    F, m, d = w.F, w.m, w.d
    x = I.draw_facts(F, d, m, seed=w.seed)
    K, V, A, G = (torch.from_numpy(x[n]).to(dev) for n in ("K", "V", "A", "G"))
    f = torch.from_numpy(x["f"]).to(dev)
    lib = ops.lib()
    nb = lib.hebbian_workspace_bytes(F, m, d)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    Bt = torch.empty((m, d), dtype=torch.float32, device=dev)
    out = torch.empty((F, d), dtype=torch.float32, device=dev)
    arg = torch.empty((F,), dtype=torch.int32, device=dev)
    st = ops._stream()
    p = ops._ptr

    def write(_):
        if lib.hebbian_write(p(K), p(V), p(f), F, F, p(A), p(G), m, d, p(Bt), p(ws), ws.numel(), st) != 0:
            raise RuntimeError(ops._lib.last_error())

    def read_recall(_):
        if lib.hebbian_read(p(K), F, p(A), p(G), p(Bt), m, d, p(out), st) != 0:
            raise RuntimeError(ops._lib.last_error())
        if lib.recall_argmax(p(out), p(V), 1, F, F, d, p(arg), None, st) != 0:
            raise RuntimeError(ops._lib.last_error())

    _, ms_w, kernel_ms = time_calls(write, steps, warmup, KernelTimer(steps))
    _, ms_r, _ = time_calls(read_recall, steps, warmup)
    torch.cuda.synchronize()
    stored = float((arg.cpu().numpy() == x["f"]).mean())
    w_flops = 6.0 * F * m * d       # two feature products, their product, the accumulation
    r_flops = 6.0 * F * m * d + 2.0 * F * F * d  # the same for the reads, then the recall scores
    return {"workload": w.name, "ms_per_step": ms_w + ms_r, "facts_per_s": F / ((ms_w + ms_r) * 1e-3),
            "roofline": roofline("mfma", w_flops / (kernel_ms * 1e-3) / 1e12, PEAK_FP32_TFLOPS, "TFLOP/s"),
            "main_kernel": {"name": "hebbian_write_kernel<128>", "ms": kernel_ms},
            "write_ms": ms_w, "read_recall_ms": ms_r,
            "read_recall_tflops": r_flops / (ms_r * 1e-3) / 1e12,
            "stored_fraction": stored,
            "config": {"F": F, "m": m, "d": d, "dtype_in": "f32"}}


def bench_capacity(dev, groups=64, d=64, W=256, ns=(32, 64, 128, 256, 512, 1024, 2048), lams=(1.0, 0.999)):
    """Recall of old pairs from the eviction-conditioned and the ingest-all
    memory as pairs pile up (every step in libtc; one untimed pass first)."""
    import numpy as np
    import torch

    from linear_attention_tensor_amd import diagnostics as Dg
    from linear_attention_tensor_amd import inputs as I

    curves = []
    t0 = time.perf_counter()
    for lam in lams:
        for n in ns:
            x = I.draw_pairs(groups, n + W, d, seed=1000 + n)
            k, v = to_dev_f32(x["k"], dev), to_dev_f32(x["v"], dev)
            lam_t, eta_t = to_dev_f32(np.full(1, lam), dev), to_dev_f32(np.ones(1), dev)
            Dg.capacity_point(k, v, lam_t, eta_t, W, n)
            torch.cuda.synchronize()
            a = time.perf_counter()
            tc_rate, ia_rate = Dg.capacity_point(k, v, lam_t, eta_t, W, n)
            torch.cuda.synchronize()
            curves.append({"lam": lam, "n_old": n, "recall_eviction_conditioned": tc_rate,
                           "recall_ingest_all": ia_rate, "ms": (time.perf_counter() - a) * 1e3})
    return {"workload": "capacity_diagnostic", "config": {"groups": groups, "d": d, "W": W, "dtype_in": "f32"},
            "curve": curves, "wall_s": time.perf_counter() - t0}


def cpu_baseline_fused(x, T_sample=16384):
    """The float64 oracle (as it stands) on a bounded prefix of the same
    input, with its BLAS pinned to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import tc as O

    w_W = 1024
    sl = (slice(None), slice(None), slice(0, T_sample))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.tc_fused(x["q64"][sl], x["k64"][sl], x["v64"][sl], x["lam"].astype(np.float64), x["eta"],
                   x["g"].astype(np.float64), w_W)
        dt = time.perf_counter() - t0
    B, H = x["q64"].shape[:2]
    return {"value": B * H * T_sample / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cores": len(os.sched_getaffinity(0)), "blas_threads": 1,
            "sample": f"fused layer oracle (NumPy float64, BLAS limited to 1 thread) on the first {T_sample} "
                      f"tokens of all {B * H} heads of the same input ({dt:.1f} s; the first {w_W} tokens "
                      f"have shorter windows)"}


class _Components(dict):
    """Component results by name; each announces itself on stderr when it is
    done, so that a long run shows its progress."""

    def __setitem__(self, key, value):
        print(f"[bench] {key} done", file=sys.stderr, flush=True)
        super().__setitem__(key, value)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(each GPU would run its own share of the heads); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                                               "copies": 2}}))
        return
    only = args.only
    components = _Components()
    if only in (None, "fused"):
        head, x = bench_fused(args.steps, args.warmup, dev)
    if only is None and not args.no_components:
        components["fused_layer_f32"] = bench_fused_f32(args.steps, args.warmup, dev, x)
        components["prefill_scan_f32"] = bench_scan(args.steps, args.warmup, dev)
        components["prefill_scan_backward_f32"] = bench_scan_backward(args.steps, args.warmup, dev)
        components["fused_layer_backward_bf16"] = bench_layer_backward(args.steps, args.warmup, dev, x)
        components["fused_layer_backward_f32"] = bench_layer_backward_f32(args.steps, args.warmup, dev)
        components["scan_bf16_fused_size"] = bench_scan_bf16(args.steps, args.warmup, dev)
        components["decode_bf16"] = bench_decode(args.steps, args.warmup, dev, n_steps=args.decode_steps or 4096)
        components["decode_bf16_x4"] = bench_decode(args.steps, args.warmup, dev, n_steps=args.decode_steps or 1024,
                                                    B=256)
        components["decode_layer_bf16"] = bench_decode_layer(args.steps, args.warmup, dev)
        components["delta_scan_bf16"] = bench_delta(args.steps, args.warmup, dev)
        components["delta_scan_f32"] = bench_delta_f32(args.steps, args.warmup, dev)
        components["delta_backward_f32"] = bench_delta_backward(args.steps, args.warmup, dev)
        components["delta_backward_bf16"] = bench_delta_backward(args.steps, args.warmup, dev, "delta_scan_bf16", True)
        components["hebbian_f32"] = bench_hebbian(args.steps, args.warmup, dev)
        components["capacity_diagnostic"] = bench_capacity(dev)
    elif only == "fused_f32":
        components["fused_layer_f32"] = bench_fused_f32(args.steps, args.warmup, dev)
    elif only == "scan":
        components["prefill_scan_f32"] = bench_scan(args.steps, args.warmup, dev)
    elif only == "scan_bf16":
        components["scan_bf16_fused_size"] = bench_scan_bf16(args.steps, args.warmup, dev)
    elif only == "scan_backward":
        components["prefill_scan_backward_f32"] = bench_scan_backward(args.steps, args.warmup, dev)
    elif only == "layer_backward":
        components["fused_layer_backward_bf16"] = bench_layer_backward(args.steps, args.warmup, dev)
        components["fused_layer_backward_f32"] = bench_layer_backward_f32(args.steps, args.warmup, dev)
    elif only == "decode":
        components["decode_bf16"] = bench_decode(args.steps, args.warmup, dev, n_steps=args.decode_steps or 4096)
    elif only == "decode_x4":
        components["decode_bf16_x4"] = bench_decode(args.steps, args.warmup, dev, n_steps=args.decode_steps or 1024,
                                                    B=256)
    elif only == "decode_layer":
        components["decode_layer_bf16"] = bench_decode_layer(args.steps, args.warmup, dev)
    elif only == "delta":
        components["delta_scan_bf16"] = bench_delta(args.steps, args.warmup, dev)
    elif only == "delta_f32":
        components["delta_scan_f32"] = bench_delta_f32(args.steps, args.warmup, dev)
    elif only == "delta_backward":
        components["delta_backward_f32"] = bench_delta_backward(args.steps, args.warmup, dev)
        components["delta_backward_bf16"] = bench_delta_backward(args.steps, args.warmup, dev, "delta_scan_bf16", True)
    elif only == "hebbian":
        components["hebbian_f32"] = bench_hebbian(args.steps, args.warmup, dev)
    elif only == "capacity":
        components["capacity_diagnostic"] = bench_capacity(dev)
    if only not in (None, "fused"):
        print(json.dumps({"only": only, "components": components}))
        return
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1/d) q,k,v with unit keys; per-head lam, eta, g)",
        "config": head["config"],
        "roofline": head["roofline"],
        "layer_roofline": head["layer_roofline"],
        "main_kernel": head["main_kernel"],
        "layer": head["layer"],
        "l2_overhead": head["l2_overhead"],
    }
    if components:
        line["components"] = components
        if "scan_bf16_fused_size" in components:
            line["memory_scan_roofline"] = dict(
                components["scan_bf16_fused_size"]["mfma"],
                scope="the L2 memory scan alone (tc_scan_forward, bf16, same sizes): its flops / call time")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_fused(x)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
