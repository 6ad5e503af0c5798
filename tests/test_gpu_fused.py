"""Parity of tc_fused_layer (C ABI, HIP kernels) against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu


def run(x, W, g=None, scale=None):
    y, A = ops.tc_fused_layer(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                              f32_dev(x["lam"]), f32_dev(x["eta"]), f32_dev(x["g"] if g is None else g), W,
                              softmax_scale=scale, return_state=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), A.cpu().numpy()


@pytest.mark.parametrize("B,H,T,d,W", [
    (1, 2, 300, 64, 64),
    (1, 2, 513, 128, 100),
    (2, 1, 200, 64, 1),
    (1, 1, 100, 128, 500),   # window covers the sequence: causal softmax, no L2
    (1, 2, 64, 64, 64),
    (1, 1, 1, 128, 4),
    (1, 3, 1100, 128, 1024),
    (1, 32, 2100, 64, 100),  # > 256 tiles: the pre-pass walks two tiles per workgroup
    (1, 32, 2100, 64, 700),  # ... with tiles that write no evictions, W % 8 != 0
])
def test_fused_small(B, H, T, d, W):
    print(f"[case] fused B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=2000 + T, dtype="bf16", lam=("uniform", 0.95, 0.999))
    y, A = run(x, W)
    y_ref, A_ref = O.tc_fused(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                              x["g"].astype(np.float64), W)
    check("y", y, y_ref, 2e-2)
    check("A", A, A_ref, 2e-2)


def test_fused_gate_closed_is_sliding_window():
    x = I.draw(1, 2, 400, 128, seed=3, dtype="bf16")
    W = 96
    y, _ = run(x, W, g=np.full(2, -1e4, np.float32), scale=0.2)
    ref = O.window_softmax(x["q64"], x["k64"], x["v64"], W, 0.2)
    check("y", y, ref, 2e-2)


def test_fused_layer_full_size_sampled_rows_and_a_whole_head():
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] fused full size", flush=True)
    x = I.draw_workload("fused_layer_bf16")
    y, A = run(x, w.W)
    rows = [0, 1, 63, 64, w.W - 1, w.W, w.W + 1, w.W + 127, 4097, 16383, 16384, 30000, w.T - 64, w.T - 1]
    ref = O.tc_fused_rows(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                          x["g"].astype(np.float64), w.W, rows)
    check("y rows", y[:, :, rows], ref, 2e-2)
    # one whole head, every row (each of its 128 tiles), and its final state
    h = 5
    y_h, A_h = O.tc_fused(x["q64"][:, h:h + 1], x["k64"][:, h:h + 1], x["v64"][:, h:h + 1],
                          x["lam"][h:h + 1].astype(np.float64), x["eta"][h:h + 1],
                          x["g"][h:h + 1].astype(np.float64), w.W)
    check(f"y head {h}", y[:, h:h + 1], y_h, 2e-2)
    check(f"A head {h}", A[:, h:h + 1], A_h, 2e-2)


@pytest.mark.parametrize("dtype,B,H,T,d,W", [
    ("f32", 1, 1, 256, 16, 32),     # the tiny single-head workload's shape
    ("f32", 2, 3, 300, 32, 17),
    ("f32", 1, 2, 1000, 64, 100),
    ("f32", 1, 1, 300, 128, 64),
    ("f32", 1, 2, 1100, 128, 333),  # the four-piece scan and several window tiles per head
    ("f32", 1, 2, 40, 16, 100),     # T < W: the L2 memory stays empty
    ("bf16", 1, 2, 300, 16, 40),
    ("bf16", 2, 1, 257, 32, 64),
])
def test_fused_fp32_and_small_d(dtype, B, H, T, d, W):
    # fp32 inputs and d in {16, 32}: the prefill scan's read, then the window
    # softmax with the gate in fp32 arithmetic
    print(f"[case] fused {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=2500 + T + d, dtype=dtype)
    y, A = ops.tc_fused_layer(*(to_dev(x[n], dtype) for n in ("q", "k", "v")), f32_dev(x["lam"]),
                              f32_dev(x["eta"]), f32_dev(x["g"]), W, return_state=True)
    torch.cuda.synchronize()
    y_ref, A_ref = O.tc_fused(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                              x["g"].astype(np.float64), W)
    tol = 1e-5 if dtype == "f32" else 2e-2
    check("y", y.cpu().numpy(), y_ref, tol)
    check("A", A.cpu().numpy(), A_ref, tol)


def test_fused_fp32_prefill_workload_sampled_rows():
    # the batched fp32 prefill workload's inputs (B=4, H=8, T=4096, d=64, W=512) through the whole layer
    w = I.WORKLOADS["prefill_scan_f32"]
    print("[case] fused fp32 at the prefill workload", flush=True)
    x = I.draw_workload(w.name)
    g = np.random.default_rng(3).standard_normal(w.H).astype(np.float32)
    y = ops.tc_fused_layer(*(to_dev(x[n], "f32") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                           f32_dev(x["eta"]), f32_dev(g), w.W).cpu().numpy()
    rows = [0, 511, 512, 513, 1000, 2047, 4095]
    ref = O.tc_fused_rows(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                          g.astype(np.float64), w.W, rows)
    check("y rows", y[:, :, rows], ref, 1e-5)


def test_fused_layer_f32_full_size_sampled_rows_and_a_whole_head():
    # the fp32-input layer at the headline shape (the bf16 workload's values held in fp32), as bench.py runs it:
    # the four-piece fp32 scan, then the fp32-MFMA window softmax with the gate
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] fused fp32 full size", flush=True)
    x = I.draw_workload("fused_layer_bf16")
    y, A = ops.tc_fused_layer(*(to_dev(x[n + "64"], "f32") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                              f32_dev(x["eta"]), f32_dev(x["g"]), w.W, return_state=True)
    torch.cuda.synchronize()
    y, A = y.cpu().numpy(), A.cpu().numpy()
    rows = [0, 1, 31, 32, w.W - 1, w.W, w.W + 1, 4097, 16383, 16384, 30000, w.T - 1]
    ref = O.tc_fused_rows(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                          x["g"].astype(np.float64), w.W, rows)
    check("y rows", y[:, :, rows], ref, 1e-5)
    h = 9
    y_h, A_h = O.tc_fused(x["q64"][:, h:h + 1], x["k64"][:, h:h + 1], x["v64"][:, h:h + 1],
                          x["lam"][h:h + 1].astype(np.float64), x["eta"][h:h + 1],
                          x["g"][h:h + 1].astype(np.float64), w.W)
    check(f"y head {h}", y[:, h:h + 1], y_h, 1e-5)
    check(f"A head {h}", A[:, h:h + 1], A_h, 1e-5)
