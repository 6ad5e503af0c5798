"""Parity of tc_decode_layer_step (C ABI, HIP kernel) against the float64 oracle.

Tensor Cache, Methodology 1: one decode step of the whole layer (eviction into
A, the new pair into the ring, exact softmax over the ring, gated L2 read).
"""
import math

import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,d,W,T", [(2, 3, 64, 8, 40), (1, 2, 128, 5, 23), (3, 1, 16, 1, 9),
                                       (1, 1, 32, 64, 70), (1, 2, 128, 37, 90)])
def test_decode_layer_from_empty_matches_fused_layer(dtype, B, H, d, W, T):
    print(f"[case] decode layer dtype={dtype} B={B} H={H} d={d} W={W} T={T}", flush=True)
    x = I.draw(B, H, T, d, seed=600 + d + W, dtype=dtype)
    scale = 1.0 / math.sqrt(d)
    y_ref, A_ref = O.tc_fused(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"], x["g"],
                              W, scale)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ring_k = torch.zeros((B, H, W, d), dtype=tdt, device="cuda")
    ring_v = torch.zeros((B, H, W, d), dtype=tdt, device="cuda")
    A = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    lam, eta, g = f32_dev(x["lam"]), f32_dev(x["eta"]), f32_dev(x["g"])
    ys = []
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        ys.append(ops.tc_decode_layer_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                           v[:, :, t].contiguous(), ring_k, ring_v, A, lam, eta, g, pos,
                                           W).clone())
    y = torch.stack(ys, dim=2).cpu().numpy()
    check("y", y, y_ref, TOL[dtype])
    check("A", A.cpu().numpy(), A_ref, TOL[dtype])
    rk = ring_k.cpu()
    kk = k.cpu()
    for t in range(max(0, T - W), T):
        assert torch.equal(rk[:, :, t % W], kk[:, :, t])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_layer_sequences_at_different_positions(dtype):
    B, H, d, W = 3, 2, 64, 6
    rng = np.random.default_rng(19)
    pos0 = np.array([0, 4, 17])
    ring_k = rng.standard_normal((B, H, W, d)) / math.sqrt(d)
    ring_v = rng.standard_normal((B, H, W, d)) / math.sqrt(d)
    A0 = rng.standard_normal((B, H, d, d)) * 0.1
    rk_s, rk64 = I.round_to_dtype(ring_k, dtype)
    rv_s, rv64 = I.round_to_dtype(ring_v, dtype)
    sc = I.decode_scalars(H)
    g = rng.standard_normal(H)
    dec = O.TensorCacheDecoder.from_state(rk64, rv64, A0.astype(np.float32).astype(np.float64), pos0, W,
                                          sc["lam"], sc["eta"])
    g_rk, g_rv, g_A = to_dev(rk_s, dtype), to_dev(rv_s, dtype), f32_dev(A0)
    lam, eta, gg = f32_dev(sc["lam"]), f32_dev(sc["eta"]), f32_dev(g)
    for step in range(12):
        x = I.draw_decode_position(B, H, d, 2000 + step, dtype=dtype)
        pos = torch.from_numpy(pos0 + step).to("cuda")
        y = ops.tc_decode_layer_step(to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype),
                                     g_rk, g_rv, g_A, lam, eta, gg, pos, W, softmax_scale=0.3)
        y_ref = dec.step_layer(x["q64"], x["k64"], x["v64"], g, 0.3)
        check(f"step {step}", y.cpu().numpy(), y_ref, TOL[dtype])
    check("A", g_A.cpu().numpy(), dec.A, TOL[dtype])


def test_decode_layer_workload_full_size_sampled_sequences():
    # 64 sequences x 32 heads, d = 128, W = 2048, bf16, full ring at pos = W, A = 0
    w = I.WORKLOADS["decode_bf16"]
    B, H, d, W = w.B, w.H, w.d, w.W
    print("[case] decode layer full size", flush=True)
    rk, rv = I.draw_ring(B, H, W, d)
    sc = I.decode_scalars(H)
    g = np.random.default_rng(7).standard_normal(H)
    g_rk, g_rv = to_dev(rk, "bf16"), to_dev(rv, "bf16")
    g_A = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    lam, eta, gg = f32_dev(sc["lam"]), f32_dev(sc["eta"]), f32_dev(g)
    bs = [0, 13, 63]
    dec = O.TensorCacheDecoder.from_state(I.storage_to_f64(rk[bs], "bf16"), I.storage_to_f64(rv[bs], "bf16"),
                                          np.zeros((len(bs), H, d, d)), np.full(len(bs), W), W,
                                          sc["lam"], sc["eta"])
    for step in range(4):
        x = I.draw_decode_position(B, H, d, W + step)
        pos = torch.full((B,), W + step, dtype=torch.int64, device="cuda")
        y = ops.tc_decode_layer_step(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                                     g_rk, g_rv, g_A, lam, eta, gg, pos, W)
        y_ref = dec.step_layer(x["q64"][bs], x["k64"][bs], x["v64"][bs], g)
        check(f"step {step}", y.cpu().numpy()[bs], y_ref, 2e-2)
    check("A", g_A.cpu().numpy()[bs], dec.A, 2e-2)
