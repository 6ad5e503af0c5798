"""Parity of tc_scan_forward (C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def run(x, W):
    dev = "cuda"
    m, A = ops.tc_scan_forward(to_dev(x["q"], x["dtype"]), to_dev(x["k"], x["dtype"]),
                               to_dev(x["v"], x["dtype"]), f32_dev(x["lam"]), f32_dev(x["eta"]), W)
    torch.cuda.synchronize()
    return m.cpu().numpy(), A.cpu().numpy()


def lam_of(x):
    return x["lam"].astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,T,d,W", [
    (1, 1, 256, 16, 32),        # the tiny single-head workload shape
    (2, 3, 300, 32, 17),        # several chunks, ragged tail
    (1, 2, 1000, 64, 100),      # many segments
    (2, 2, 777, 128, 64),       # d=128 (fp32: four d=64 pieces, the second column half of q, k added)
    (1, 2, 3000, 128, 200),     # d=128, many segments per piece
    (1, 2, 130, 128, 1),        # d=128, W = 1
    (1, 1, 40, 128, 100),       # d=128, T < W: m and the final state are zero
    (1, 1, 64 + 10, 64, 10),    # exactly one full chunk of active rows
    (1, 2, 40, 16, 1),          # W = 1
    (1, 1, 30, 16, 30),         # T == W: nothing is evicted
    (1, 1, 20, 32, 45),         # T < W
])
def test_scan_small(dtype, B, H, T, d, W):
    print(f"[case] scan dtype={dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=1000 + T + d, dtype=dtype)
    m, A = run(x, W)
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], lam_of(x), x["eta"], W)
    check("m", m, m_ref, TOL[dtype])
    check("A", A, A_ref, TOL[dtype])
    assert np.all(m[:, :, : min(W, T)] == 0.0)


@pytest.mark.parametrize("lam_val", [0.0, 1.0])
def test_scan_lambda_edges(lam_val):
    x = I.draw(1, 2, 333, 64, seed=77, dtype="f32", lam=("fixed", lam_val))
    m, A = run(x, 20)
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], lam_of(x), x["eta"], 20)
    check(f"m lam={lam_val}", m, m_ref, 1e-5)
    check(f"A lam={lam_val}", A, A_ref, 1e-5)


def test_scan_empty_sequence():
    x = I.draw(1, 2, 1, 64, seed=5, dtype="f32")
    q = to_dev(x["q"], "f32")[:, :, :0].contiguous()
    m, A = ops.tc_scan_forward(q, q.clone(), q.clone(), f32_dev(x["lam"]), f32_dev(x["eta"]), 8)
    torch.cuda.synchronize()
    assert m.shape == (1, 2, 0, 64)
    assert torch.all(A == 0)


@pytest.mark.parametrize("name", ["tiny_scan_f32", "prefill_scan_f32"])
def test_scan_workloads_full_size(name):
    w = I.WORKLOADS[name]
    print(f"[case] scan workload {name}", flush=True)
    x = I.draw_workload(name)
    m, A = run(x, w.W)
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], lam_of(x), x["eta"], w.W)
    check(f"{name} m", m, m_ref, TOL[w.dtype])
    check(f"{name} A", A, A_ref, TOL[w.dtype])


def test_scan_fused_size_bf16_sampled_rows():
    # the bf16 scan at the fused-layer size (H=16, T=32768, W=1024, d=128), spot rows
    w = I.WORKLOADS["fused_layer_bf16"]
    print("[case] scan bf16 at the fused-layer size", flush=True)
    x = I.draw_workload("fused_layer_bf16")
    m, A = run(x, w.W)
    rows = [0, w.W - 1, w.W, w.W + 1, w.W + 63, w.W + 64, 5000, 16384, 20001, w.T - 65, w.T - 1]
    ref = O.tc_scan_rows(x["q64"], x["k64"], x["v64"], lam_of(x), x["eta"], w.W, rows)
    check("m rows", m[:, :, rows], ref, 2e-2)


@pytest.mark.parametrize("B,H,T,d,W", [
    (1, 2, 300, 128, 1),       # W = 1
    (2, 1, 100, 64, 150),      # T < W: nothing evicted
    (1, 1, 257, 128, 256),     # one eviction
    (1, 3, 1000, 64, 300),     # several tiles, W not a multiple of 8
    (2, 2, 2049, 128, 1024),   # many tiles, ragged last tile
    (1, 1, 513, 64, 7),
    # more (tile, b, h) units than the read kernel's persistent grid (256
    # workgroups at d = 128, 512 at d = 64): some workgroups take a second
    # unit, with its K rows loaded during the first
    (1, 3, 256 * 90 + 77, 128, 1000),
    (2, 2, 256 * 130 + 5, 64, 64),
])
def test_scan_bf16_tiled_path(B, H, T, d, W):
    # bf16 inputs with d in {64, 128} run on the fused layer's pre-pass and
    # prefix plus the L2-read kernel (256-query chunks)
    print(f"[case] scan bf16 tiled B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=5000 + T + W, dtype="bf16", lam=("uniform", 0.95, 0.999))
    m, A = run(x, W)
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], lam_of(x), x["eta"], W)
    check("m", m, m_ref, 2e-2)
    check("A", A, A_ref, 2e-2)
    assert np.all(m[:, :, : min(W, T)] == 0.0)
