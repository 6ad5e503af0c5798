"""Parity of tc_fused_layer (C ABI, HIP kernels) against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, report, to_dev

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
    assert report("y", y, y_ref) <= 2e-2
    assert report("A", A, A_ref) <= 2e-2


def test_fused_gate_closed_is_sliding_window():
    x = I.draw(1, 2, 400, 128, seed=3, dtype="bf16")
    W = 96
    y, _ = run(x, W, g=np.full(2, -1e4, np.float32), scale=0.2)
    ref = O.window_softmax(x["q64"], x["k64"], x["v64"], W, 0.2)
    assert report("y", y, ref) <= 2e-2


def test_fused_layer_full_size_sampled_rows():
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] fused full size", flush=True)
    x = I.draw_workload("fused_layer_bf16")
    y, A = run(x, w.W)
    rows = [0, 1, 63, 64, w.W - 1, w.W, w.W + 1, w.W + 127, 4097, 16383, 16384, 30000, w.T - 64, w.T - 1]
    ref = O.tc_fused_rows(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"],
                          x["g"].astype(np.float64), w.W, rows)
    assert report("y rows", y[:, :, rows], ref) <= 2e-2
