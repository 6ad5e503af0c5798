"""tc_scan_forward_noalloc (the entry point for callers that cannot allocate)
against tc_scan_forward with a caller workspace: the same kernels on the
same inputs, so the same bits, and the oracle's bar besides.  Two calls in
a row, the second smaller, so the second runs on scratch the first left
behind.  Called through the C ABI (ctypes)."""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import _lib
from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import check, f32_dev, same_bits, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def noalloc(q, k, v, lam, eta, W, m, A):
    B, H, T, d = q.shape
    dt = _lib.TC_BF16 if q.dtype == torch.bfloat16 else _lib.TC_F32
    st = _lib.lib().tc_scan_forward_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), dt,
        ctypes.c_void_p(lam.data_ptr()), ctypes.c_void_p(eta.data_ptr()), B, H, T, d, d, W, 64,
        ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(A.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def one_case(dtype, B, H, T, d, W, seed, heads):
    print(f"[case] noalloc {dtype} B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=seed, dtype=dtype)
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    lam, eta = f32_dev(x["lam"]), f32_dev(x["eta"])
    m = torch.full((B, H, T, d), float("nan"), dtype=torch.float32, device="cuda")
    A = torch.full((B, H, d, d), float("nan"), dtype=torch.float32, device="cuda")
    assert noalloc(q, k, v, lam, eta, W, m, A) == _lib.TC_OK, _lib.last_error()
    m_ws, A_ws = ops.tc_scan_forward(q, k, v, lam, eta, W)
    torch.cuda.synchronize()
    same_bits("m vs tc_scan_forward", m, m_ws)
    same_bits("A vs tc_scan_forward", A, A_ws)
    sl = (slice(None), heads)
    m_ref, A_ref = O.tc_scan(x["q64"][sl], x["k64"][sl], x["v64"][sl], x["lam"][heads].astype(np.float64),
                             x["eta"][heads], W)
    check("m vs oracle", m.cpu().numpy()[sl], m_ref, TOL[dtype])
    check("A vs oracle", A.cpu().numpy()[sl], A_ref, TOL[dtype])


def test_noalloc_two_calls_second_smaller():
    # the batched fp32 prefill workload (4 MiB of segment states), then a
    # smaller call that reuses the scratch the first one wrote
    one_case("f32", 4, 8, 4096, 64, 512, seed=102, heads=[0, 5])
    one_case("f32", 2, 3, 700, 32, 50, seed=71, heads=[0, 1, 2])


def test_noalloc_bf16_tiled_then_smaller():
    # bf16 d = 128 runs on the per-tile state path (4 MiB at this size)
    one_case("bf16", 1, 4, 4096, 128, 512, seed=72, heads=[1, 3])
    one_case("bf16", 1, 2, 1000, 64, 100, seed=73, heads=[0, 1])


def test_noalloc_rejects_calls_beyond_the_scratch():
    # bf16 d = 128, 8 heads of 32768 tokens: 64 MiB of tile states > 32 MiB
    B, H, T, d, W = 1, 8, 32768, 128, 1024
    need = ops.scan_workspace(B, H, T, d, d, W, _lib.TC_BF16)
    assert need > 32 << 20
    q = torch.zeros((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    lam = torch.full((H,), 0.9, dtype=torch.float32, device="cuda")
    m = torch.zeros((B, H, T, d), dtype=torch.float32, device="cuda")
    A = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    st = noalloc(q, q, q, lam, lam, W, m, A)
    assert st == _lib.TC_ERR_WORKSPACE
    assert "scratch" in _lib.last_error()
