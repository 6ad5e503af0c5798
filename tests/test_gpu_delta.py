"""Parity of delta_scan_forward (C ABI, HIP kernel) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import delta as D
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def run(x, S0=None):
    o, S = ops.delta_scan_forward(to_dev(x["q"], x["dtype"]), to_dev(x["k"], x["dtype"]),
                                  to_dev(x["v"], x["dtype"]), f32_dev(x["beta"]),
                                  S0=None if S0 is None else f32_dev(S0), return_state=True)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,T,d,with_s0", [
    (1, 2, 200, 64, False),
    (2, 1, 130, 128, True),
    (1, 1, 64, 16, False),
    (1, 2, 1, 32, True),
    (1, 1, 257, 128, False),
    # one ragged chunk (T < 64) and a full chunk plus a ragged one, at the
    # widths of the bf16 LDS-DMA kernel
    (1, 2, 1, 64, False),
    (1, 2, 40, 64, True),
    (2, 1, 100, 64, False),
    (1, 2, 1, 128, True),
    (1, 2, 40, 128, False),
    (2, 1, 100, 128, True),
])
def test_delta_small(dtype, B, H, T, d, with_s0):
    print(f"[case] delta dtype={dtype} B={B} H={H} T={T} d={d} S0={with_s0}", flush=True)
    x = I.draw(B, H, T, d, seed=4000 + T + d, dtype=dtype)
    S0 = (np.random.default_rng(1).standard_normal((B, H, d, d)) * 0.2).astype(np.float32) if with_s0 else None
    o, S = run(x, S0)
    o_ref, S_ref = D.delta_scan(x["q64"], x["k64"], x["v64"], x["beta"].astype(np.float64),
                                None if S0 is None else S0.astype(np.float64))
    check("o", o, o_ref, TOL[dtype])
    check("S", S, S_ref, TOL[dtype])


def test_delta_beta_one_rereads_value():
    # beta = 1 and q_t = k_t: the read after the write returns v_t
    x = I.draw(1, 2, 150, 64, seed=8, dtype="f32")
    x["q"] = x["k"].copy()
    x["beta"] = np.ones_like(x["beta"])
    o, _ = run(x)
    check("o vs v", o, x["v64"], 1e-5)


def test_delta_workload_full_size_sampled_heads():
    w = I.WORKLOADS["delta_scan_bf16"]
    print("[case] delta full size", flush=True)
    x = I.draw_workload("delta_scan_bf16")
    o, S = run(x)
    hs = [0, 7, 15]
    sl = (slice(None), hs)
    o_ref, S_ref = D.delta_scan(x["q64"][sl], x["k64"][sl], x["v64"][sl], x["beta"][sl].astype(np.float64))
    check("o", o[sl], o_ref, 2e-2)
    check("S", S[sl], S_ref, 2e-2)
