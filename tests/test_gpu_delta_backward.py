"""Parity of delta_scan_backward (C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import delta as D
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2  # the bar for bf16 inputs
NAMES = ("dq", "dk", "dv", "dbeta", "dS0")


def run(x, do, S0=None, dSf=None):
    g = ops.delta_scan_backward(to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
                                f32_dev(x["beta"]), f32_dev(do), S0=None if S0 is None else f32_dev(S0),
                                dS_final=None if dSf is None else f32_dev(dSf), return_dS0=True)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in g]


def ref(x, do, S0=None, dSf=None):
    f = (lambda a: None if a is None else np.asarray(a, np.float64))
    return D.delta_scan_backward(x["q64"], x["k64"], x["v64"], x["beta"].astype(np.float64),
                                 do.astype(np.float64), f(S0), f(dSf))


@pytest.mark.parametrize("B,H,T,d,states", [
    (1, 1, 64, 16, False),     # one full chunk
    (1, 2, 200, 64, False),    # ragged tail
    (2, 1, 130, 32, True),     # initial state and final-state cotangent
    (1, 1, 1, 16, True),       # one token
    (1, 2, 37, 64, True),      # shorter than a chunk
    (2, 2, 513, 64, False),    # many chunks
    (1, 3, 300, 16, True),
    # d = 128: the gradient kernel walks the state rows in pieces of 16
    (1, 1, 64, 128, True),
    (1, 2, 200, 128, False),
    (2, 1, 37, 128, True),
    (1, 1, 1, 128, True),
    (1, 1, 300, 128, True),
])
def test_delta_backward_small(B, H, T, d, states):
    print(f"[case] delta backward B={B} H={H} T={T} d={d} states={states}", flush=True)
    x = I.draw(B, H, T, d, seed=6000 + T + d, dtype="f32")
    do = I.draw_cotangent(B, H, T, d, seed=6000 + T + d)
    rng = np.random.default_rng(T + d)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.2).astype(np.float32) if states else None
    dSf = (rng.standard_normal((B, H, d, d)) * 0.2).astype(np.float32) if states else None
    got = run(x, do, S0, dSf)
    want = ref(x, do, S0, dSf)
    for name, a, b in zip(NAMES, got, want):
        check(name, a, b, TOL)


@pytest.mark.parametrize("beta_val", [0.0, 1.0])
def test_delta_backward_beta_edges(beta_val):
    print(f"[case] delta backward beta={beta_val}", flush=True)
    x = I.draw(1, 2, 150, 32, seed=81, dtype="f32")
    x["beta"] = np.full_like(x["beta"], beta_val)
    do = I.draw_cotangent(1, 2, 150, 32, seed=81)
    S0 = (np.random.default_rng(82).standard_normal((1, 2, 32, 32)) * 0.2).astype(np.float32)
    got = run(x, do, S0)
    want = ref(x, do, S0)
    for name, a, b in zip(NAMES, got, want):
        check(f"beta={beta_val} {name}", a, b, TOL)


def test_delta_backward_empty_sequence():
    x = I.draw(1, 2, 1, 16, seed=5, dtype="f32")
    q = to_dev(x["q"], "f32")[:, :, :0].contiguous()
    dSf = torch.randn(1, 2, 16, 16, device="cuda")
    g = ops.delta_scan_backward(q, q.clone(), q.clone(), torch.zeros(1, 2, 0, device="cuda"), q.clone(),
                                dS_final=dSf, return_dS0=True)
    torch.cuda.synchronize()
    assert g[0].shape == (1, 2, 0, 16)
    assert torch.equal(g[4], dSf)


@pytest.mark.parametrize("d", [64, 128])
def test_delta_backward_repeat_is_deterministic(d):
    x = I.draw(1, 2, 700, d, seed=9, dtype="f32")
    do = I.draw_cotangent(1, 2, 700, d, seed=9)
    a = run(x, do)
    b = run(x, do)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_delta_backward_full_size_sampled_heads():
    # B=2 H=16 T=16384 d=64: the oracle on two whole heads (every b, t)
    w = I.WORKLOADS["delta_backward_f32"]
    print("[case] delta backward full size", flush=True)
    x = I.draw_workload("delta_backward_f32")
    do = I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed)
    got = run(x, do)
    for b, h in ((0, 0), (1, 11)):
        xs = {n: x[n][b:b + 1, h:h + 1] for n in ("q64", "k64", "v64", "beta")}
        want = D.delta_scan_backward(xs["q64"], xs["k64"], xs["v64"], xs["beta"].astype(np.float64),
                                     do[b:b + 1, h:h + 1].astype(np.float64))
        for name, a, r in zip(NAMES, got, want):
            check(f"b={b} h={h} {name}", a[b:b + 1, h:h + 1], r, TOL)


@pytest.mark.parametrize("B,H,T,d,states", [
    (1, 2, 200, 64, False),
    (2, 1, 130, 32, True),
    (1, 1, 37, 16, True),
    (1, 2, 150, 128, True),
])
def test_delta_backward_bf16_inputs(B, H, T, d, states):
    # bf16 q, k, v are widened to fp32 in the workspace: the gradients are those
    # of the bf16 values, held to the bar for bf16 inputs
    print(f"[case] delta backward bf16 B={B} H={H} T={T} d={d} states={states}", flush=True)
    x = I.draw(B, H, T, d, seed=6100 + T + d, dtype="bf16")
    do = I.draw_cotangent(B, H, T, d, seed=6100 + T + d)
    rng = np.random.default_rng(T + d + 1)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.2).astype(np.float32) if states else None
    dSf = (rng.standard_normal((B, H, d, d)) * 0.2).astype(np.float32) if states else None
    g = ops.delta_scan_backward(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), f32_dev(x["beta"]), f32_dev(do),
                                S0=None if S0 is None else f32_dev(S0),
                                dS_final=None if dSf is None else f32_dev(dSf), return_dS0=True)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, [t.cpu().numpy() for t in g], ref(x, do, S0, dSf)):
        check(name, a, b, TOL_BF16)


def test_delta_backward_bf16_workload_full_size_sampled_head():
    # the delta-rule workload itself (B=2 H=16 T=16384 d=128, bf16 inputs):
    # the oracle on one whole head (every t)
    w = I.WORKLOADS["delta_scan_bf16"]
    print("[case] delta backward bf16 workload full size", flush=True)
    x = I.draw_workload("delta_scan_bf16")
    do = I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed)
    g = ops.delta_scan_backward(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), f32_dev(x["beta"]), f32_dev(do),
                                return_dS0=True)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in g]
    b, h = 1, 5
    xs = {n: x[n][b:b + 1, h:h + 1] for n in ("q64", "k64", "v64", "beta")}
    want = D.delta_scan_backward(xs["q64"], xs["k64"], xs["v64"], xs["beta"].astype(np.float64),
                                 do[b:b + 1, h:h + 1].astype(np.float64))
    for name, a, r in zip(NAMES, got, want):
        check(f"b={b} h={h} {name}", a[b:b + 1, h:h + 1], r, TOL_BF16)
