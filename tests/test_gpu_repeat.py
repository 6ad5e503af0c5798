"""Every forward entry point, called twice on the same inputs, returns the
same bits.  No kernel uses atomics or a data-dependent order, so a
difference between two identical calls can only come from a race (a copy
landing in the wrong LDS slot, a missing wait): a mistake that a tolerance
check against the oracle could average away.  The shapes span several
tiles, chunks and workgroups per CU."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from tests._helpers import f32_dev, same_bits, to_dev

pytestmark = pytest.mark.gpu

REPEATS = 3


def dev_inputs(x):
    return tuple(to_dev(x[n], x["dtype"]) for n in ("q", "k", "v"))


@pytest.mark.parametrize("B,H,T,d,W", [(1, 16, 4096, 128, 1024), (2, 8, 3000, 64, 300)])
def test_fused_layer_repeat(B, H, T, d, W):
    print(f"[case] fused repeat B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=61 + d, dtype="bf16", lam=("uniform", 0.95, 0.999))
    q, k, v = dev_inputs(x)
    lam, eta, g = f32_dev(x["lam"]), f32_dev(x["eta"]), f32_dev(x["g"])
    first = ops.tc_fused_layer(q, k, v, lam, eta, g, W, return_state=True)
    for _ in range(REPEATS - 1):
        again = ops.tc_fused_layer(q, k, v, lam, eta, g, W, return_state=True)
        same_bits("y", first[0], again[0])
        same_bits("A_final", first[1], again[1])


@pytest.mark.parametrize("dtype,B,H,T,d,W", [
    ("f32", 4, 8, 4096, 64, 512),     # segmented fp32 MFMA scan
    ("f32", 1, 4, 2000, 128, 100),    # d = 128 fp32: four d = 64 pieces
    ("bf16", 1, 16, 8192, 128, 1024),  # pre-pass + prefix + L2-read kernel
    ("bf16", 2, 4, 3000, 32, 64),     # bf16 inputs on the d <= 64 kernels
])
def test_scan_repeat(dtype, B, H, T, d, W):
    print(f"[case] scan repeat {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=62 + d, dtype=dtype)
    q, k, v = dev_inputs(x)
    lam, eta = f32_dev(x["lam"]), f32_dev(x["eta"])
    first = ops.tc_scan_forward(q, k, v, lam, eta, W)
    for _ in range(REPEATS - 1):
        again = ops.tc_scan_forward(q, k, v, lam, eta, W)
        same_bits("m", first[0], again[0])
        same_bits("A_final", first[1], again[1])


@pytest.mark.parametrize("dtype,B,H,T,d", [
    ("bf16", 2, 16, 2048, 128),  # chunk prep + the sliced chunk walk (LDS-DMA copies)
    ("bf16", 2, 8, 1000, 64),
    ("bf16", 1, 4, 100, 128),    # one full and one ragged chunk
    ("f32", 2, 8, 1500, 64),     # fp32 prep + walk
    ("f32", 1, 2, 300, 128),
    ("bf16", 1, 2, 300, 32),
])
def test_delta_repeat(dtype, B, H, T, d):
    print(f"[case] delta repeat {dtype} B={B} H={H} T={T} d={d}", flush=True)
    x = I.draw(B, H, T, d, seed=63 + d, dtype=dtype)
    q, k, v = dev_inputs(x)
    beta = f32_dev(x["beta"])
    first = ops.delta_scan_forward(q, k, v, beta, return_state=True)
    for _ in range(REPEATS - 1):
        again = ops.delta_scan_forward(q, k, v, beta, return_state=True)
        same_bits("o", first[0], again[0])
        same_bits("S_final", first[1], again[1])


@pytest.mark.parametrize("layer", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_repeat(layer, dtype):
    # 16 sequences x 8 heads, d = 128, W = 256, past the window: every step evicts
    B, H, d, W = 16, 8, 128, 256
    print(f"[case] decode repeat layer={layer} {dtype}", flush=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rk0, rv0 = (to_dev(r, dtype) for r in I.draw_ring(B, H, W, d, dtype=dtype))
    sc = I.decode_scalars(H)
    lam, eta = f32_dev(sc["lam"]), f32_dev(sc["eta"])
    g = f32_dev(np.random.default_rng(6).standard_normal(H))
    A0 = torch.from_numpy((np.random.default_rng(5).standard_normal((B, H, d, d)) * 0.05)
                          .astype(np.float32)).cuda()
    steps = [I.draw_decode_position(B, H, d, W + s, dtype=dtype) for s in range(4)]

    def run():
        rk, rv, A = rk0.clone(), rv0.clone(), A0.clone()
        outs = []
        for s, xs in enumerate(steps):
            q, k, v = (to_dev(xs[n], dtype) for n in ("q", "k", "v"))
            pos = torch.full((B,), W + s, dtype=torch.int64, device="cuda")
            if layer:
                outs.append(ops.tc_decode_layer_step(q, k, v, rk, rv, A, lam, eta, g, pos, W).clone())
            else:
                outs.append(ops.tc_decode_step(q, k, v, rk, rv, A, lam, eta, pos, W).clone())
        return torch.stack(outs), A, rk, rv

    first = run()
    assert first[2].dtype == tdt
    for _ in range(REPEATS - 1):
        again = run()
        for name, a, b in zip(("out", "A", "ring_k", "ring_v"), first, again):
            same_bits(name, a, b)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 16)])
def test_window_and_fp32_layer_repeat(dtype, d):
    B, H, T, W = 1, 4, 2000, 300
    print(f"[case] window / layer repeat {dtype} d={d}", flush=True)
    x = I.draw(B, H, T, d, seed=64 + d, dtype=dtype)
    q, k, v = dev_inputs(x)
    lam, eta, g = f32_dev(x["lam"]), f32_dev(x["eta"]), f32_dev(x["g"])
    first = (ops.tc_window_attention(q, k, v, W), ops.tc_fused_layer(q, k, v, lam, eta, g, W))
    for _ in range(REPEATS - 1):
        again = (ops.tc_window_attention(q, k, v, W), ops.tc_fused_layer(q, k, v, lam, eta, g, W))
        same_bits("window y", first[0], again[0])
        same_bits("layer y", first[1], again[1])
