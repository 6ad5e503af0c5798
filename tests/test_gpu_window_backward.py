"""Parity of tc_window_attention_backward and tc_fused_layer_backward (C ABI,
HIP kernels) against the float64 oracle's reverse mode (pinned by central
differences and torch autograd in tests/test_oracle_window_backward.py)."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import check, f32_dev, same_bits, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dtype,B,H,T,d,W", [
    ("f32", 1, 1, 256, 16, 32),     # the tiny single-head workload's shape
    ("f32", 2, 3, 300, 32, 17),
    ("f32", 1, 2, 500, 64, 100),
    ("f32", 1, 1, 200, 128, 300),   # the window covers the sequence
    ("f32", 1, 2, 130, 64, 1),
    ("f32", 2, 2, 700, 128, 150),   # several 128-row tiles per head, W not a multiple of the 32-row block
    ("f32", 1, 1, 300, 16, 1000),   # W > T
    ("bf16", 1, 2, 400, 128, 150),
    ("bf16", 2, 1, 257, 64, 64),
    # bf16 with d in {64, 128} runs the MFMA kernels: ragged single tile, a
    # window covering the sequence, several tiles of both kernels with B > 1,
    # and the fused layer's window over many tiles
    ("bf16", 1, 2, 70, 128, 2),
    ("bf16", 1, 1, 200, 64, 300),
    ("bf16", 2, 2, 700, 128, 256),
    ("bf16", 1, 1, 3000, 128, 1024),
])
def test_window_backward(dtype, B, H, T, d, W):
    print(f"[case] window backward {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=8000 + T + d, dtype=dtype)
    dy = I.draw_cotangent(B, H, T, d, seed=8000 + T + d)
    got = ops.tc_window_attention_backward(*(to_dev(x[n], dtype) for n in ("q", "k", "v")), W, f32_dev(dy))
    torch.cuda.synchronize()
    ref = O.window_softmax_backward(x["q64"], x["k64"], x["v64"], W, 1.0 / np.sqrt(d), dy.astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        check(name, a.cpu().numpy(), b, TOL[dtype])


@pytest.mark.parametrize("dtype,B,H,T,d,W", [
    ("f32", 1, 1, 256, 16, 32),
    ("f32", 2, 2, 300, 32, 17),
    ("f32", 1, 2, 700, 64, 100),
    ("f32", 1, 1, 40, 16, 100),     # T < W: only the window branch
    ("bf16", 1, 2, 400, 64, 64),
    ("f32", 1, 2, 500, 128, 80),    # d = 128: the L2 branch in four d = 64 pieces
    ("bf16", 1, 1, 300, 128, 64),
])
def test_fused_layer_backward(dtype, B, H, T, d, W):
    print(f"[case] fused backward {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=8500 + T + d, dtype=dtype)
    dy = I.draw_cotangent(B, H, T, d, seed=8500 + T + d)
    got = ops.tc_fused_layer_backward(*(to_dev(x[n], dtype) for n in ("q", "k", "v")), f32_dev(x["lam"]),
                                      f32_dev(x["eta"]), f32_dev(x["g"]), W, f32_dev(dy))
    torch.cuda.synchronize()
    ref = O.tc_fused_backward(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64),
                              x["eta"].astype(np.float64), x["g"].astype(np.float64), W, dy.astype(np.float64))
    # per-head sums over long sequences (dlam) are held to the bf16 bar for bf16 inputs, as the read's backward
    for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta", "dg"), got, ref):
        check(name, a.cpu().numpy(), b, TOL[dtype])


def test_window_backward_repeat_is_deterministic():
    x = I.draw(1, 4, 1500, 64, seed=81, dtype="bf16")
    dy = f32_dev(I.draw_cotangent(1, 4, 1500, 64, seed=81))
    args = [to_dev(x[n], "bf16") for n in ("q", "k", "v")]
    a = ops.tc_window_attention_backward(*args, 200, dy)
    b = ops.tc_window_attention_backward(*args, 200, dy)
    for name, u, w in zip(("dq", "dk", "dv"), a, b):
        same_bits(name, u, w)


def test_fused_layer_backward_f32_prefill_workload_two_heads():
    # the fp32 layer backward at the batched prefill shape (B=4, H=8, T=4096, d=64, W=512), as bench.py runs it;
    # heads 0 and 5 of every sequence against the oracle (the per-head sums over the whole batch)
    w = I.WORKLOADS["prefill_scan_f32"]
    print("[case] fused backward fp32 prefill workload", flush=True)
    x = I.draw_workload(w.name)
    g = np.random.default_rng(3).standard_normal(w.H).astype(np.float32)
    dy = I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed)
    got = ops.tc_fused_layer_backward(*(to_dev(x[n], "f32") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                                      f32_dev(x["eta"]), f32_dev(g), w.W, f32_dev(dy))
    torch.cuda.synchronize()
    hs = [0, 5]
    sl = (slice(None), hs)
    ref = O.tc_fused_backward(x["q64"][sl], x["k64"][sl], x["v64"][sl], x["lam"][hs].astype(np.float64),
                              x["eta"][hs].astype(np.float64), g[hs].astype(np.float64), w.W,
                              dy[sl].astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check(name, a.cpu().numpy()[sl], b, 1e-5)
    for name, a, b in zip(("dlam", "deta", "dg"), got[3:], ref[3:]):
        check(name, a.cpu().numpy()[hs], b, 1e-5)


def test_fused_layer_backward_bf16_full_size_one_head():
    # the whole layer's backward at the headline size (B=1, H=16, T=32768, d=128, W=1024, bf16), as bench.py
    # runs it; one whole head (every row of dq, dk, dv and its dlam, deta, dg) against the oracle
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] fused backward bf16 full size", flush=True)
    x = I.draw_workload(w.name)
    dy = I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed)
    got = ops.tc_fused_layer_backward(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                                      f32_dev(x["eta"]), f32_dev(x["g"]), w.W, f32_dev(dy))
    torch.cuda.synchronize()
    h = 3
    sl = (slice(None), slice(h, h + 1))
    ref = O.tc_fused_backward(x["q64"][sl], x["k64"][sl], x["v64"][sl], x["lam"][h:h + 1].astype(np.float64),
                              x["eta"][h:h + 1].astype(np.float64), x["g"][h:h + 1].astype(np.float64), w.W,
                              dy[sl].astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check(f"{name} head {h}", a.cpu().numpy()[sl], b, TOL["bf16"])
    for name, a, b in zip(("dlam", "deta", "dg"), got[3:], ref[3:]):
        check(f"{name} head {h}", a.cpu().numpy()[h:h + 1], b, TOL["bf16"])
