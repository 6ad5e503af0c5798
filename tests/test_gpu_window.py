"""Parity of tc_window_attention (the L1 cache alone: exact softmax over the
W most recent tokens; C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import check, f32_dev, same_bits, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def run(x, W, scale=None):
    y = ops.tc_window_attention(*(to_dev(x[n], x["dtype"]) for n in ("q", "k", "v")), W, softmax_scale=scale)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("dtype,B,H,T,d,W", [
    ("bf16", 1, 2, 300, 64, 64),      # bf16 MFMA kernel
    ("bf16", 1, 2, 513, 128, 100),
    ("bf16", 2, 1, 200, 64, 1),
    ("bf16", 1, 1, 100, 128, 500),    # the window covers the sequence: causal softmax
    ("bf16", 1, 3, 1100, 128, 1024),
    ("bf16", 1, 2, 300, 16, 40),      # fp32-arithmetic kernel
    ("bf16", 2, 1, 257, 32, 64),
    ("f32", 1, 1, 256, 16, 32),       # the tiny single-head workload's shape
    ("f32", 2, 3, 300, 32, 17),
    ("f32", 1, 2, 500, 64, 100),
    ("f32", 1, 1, 200, 128, 300),
    ("f32", 1, 2, 130, 64, 1),
    ("f32", 2, 2, 1000, 128, 300),    # several 128-query tiles per head, W not a multiple of the 32-key block
    ("f32", 1, 3, 777, 16, 1500),     # W > T: causal softmax over the whole prefix
])
def test_window_small(dtype, B, H, T, d, W):
    print(f"[case] window {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=7000 + T + d, dtype=dtype)
    y = run(x, W)
    ref = O.window_softmax(x["q64"], x["k64"], x["v64"], W, 1.0 / np.sqrt(d))
    check("y", y, ref, TOL[dtype])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 32), ("bf16", 16), ("f32", 16), ("f32", 64), ("f32", 128)])
def test_window_one_token_returns_v(dtype, d):
    # W = 1: each query sees only its own token, whose softmax weight is 1
    x = I.draw(1, 2, 150, d, seed=71, dtype=dtype)
    y = run(x, 1)
    assert np.array_equal(y, x["v64"].astype(np.float32))


def test_window_matches_closed_gate_layer():
    # the fused layer with its gate closed is the window softmax
    x = I.draw(1, 2, 700, 128, seed=72, dtype="bf16")
    W = 200
    y_win = ops.tc_window_attention(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), W)
    y_lay = ops.tc_fused_layer(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                               f32_dev(x["eta"]), f32_dev(np.full(2, -1e4)), W)
    same_bits("window vs fused layer with the gate closed", y_win, y_lay)


def test_window_full_size_sampled_rows_and_a_whole_head():
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] window full size", flush=True)
    x = I.draw_workload("fused_layer_bf16")
    y = run(x, w.W)
    rows = [0, 1, 63, 1023, 1024, 4097, 16384, 30000, w.T - 1]
    ref = O.window_softmax_rows(x["q64"], x["k64"], x["v64"], w.W, 1.0 / np.sqrt(w.d), rows)
    check("y rows", y[:, :, rows], ref, 2e-2)
    # one whole head, every row
    h = 11
    ref_h = O.window_softmax(x["q64"][:, h:h + 1], x["k64"][:, h:h + 1], x["v64"][:, h:h + 1], w.W,
                             1.0 / np.sqrt(w.d))
    check(f"y head {h}", y[:, h:h + 1], ref_h, 2e-2)
