"""Parity of tc_scan_backward (C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2  # the bar for bf16 inputs


def run(x, W, dm):
    g = ops.tc_scan_backward(to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
                             f32_dev(x["lam"]), f32_dev(x["eta"]), W, f32_dev(dm))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in g]


def check_case(x, W, dm, label):
    got = run(x, W, dm)
    ref = O.tc_scan_backward(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64),
                             x["eta"].astype(np.float64), W, dm.astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta"), got, ref):
        check(f"{label} {name}", a, b, TOL)
    T = x["q"].shape[2]
    gq, gk, gv = got[:3]
    assert np.all(gq[:, :, : min(W, T)] == 0.0)
    assert np.all(gk[:, :, max(T - W, 0):] == 0.0)
    assert np.all(gv[:, :, max(T - W, 0):] == 0.0)
    return got


@pytest.mark.parametrize("B,H,T,d,W", [
    (1, 1, 256, 16, 32),
    (2, 3, 300, 32, 17),        # several chunks, ragged tail
    (1, 2, 1000, 64, 100),      # several segments
    (1, 1, 64 + 10, 64, 10),    # exactly one chunk of active rows
    (2, 2, 131, 64, 1),         # W = 1
    (1, 2, 40, 16, 39),         # one eviction
    (1, 1, 30, 16, 30),         # T == W: nothing is evicted
    (1, 1, 20, 32, 45),         # T < W
    (1, 2, 700, 128, 60),       # d = 128: four d = 64 pieces, gradients added
    (2, 1, 150, 128, 149),      # d = 128, one eviction
    (1, 1, 90, 128, 100),       # d = 128, T < W
    (2, 2, 1500, 128, 200),     # d = 128, many segments: the four pieces' segment states in one launch per kind
])
def test_scan_backward_small(B, H, T, d, W):
    print(f"[case] scan backward B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=4000 + T + d, dtype="f32")
    dm = I.draw_cotangent(B, H, T, d, seed=4000 + T + d)
    check_case(x, W, dm, "small")


@pytest.mark.parametrize("lam_val", [0.0, 1.0, 0.5])
def test_scan_backward_lambda_edges(lam_val):
    print(f"[case] scan backward lam={lam_val}", flush=True)
    x = I.draw(2, 2, 333, 64, seed=78, dtype="f32", lam=("fixed", lam_val))
    dm = I.draw_cotangent(2, 2, 333, 64, seed=78)
    check_case(x, 20, dm, f"lam={lam_val}")


@pytest.mark.parametrize("d", [64, 128])
def test_scan_backward_empty_sequence(d):
    x = I.draw(1, 2, 1, d, seed=5, dtype="f32")
    q = to_dev(x["q"], "f32")[:, :, :0].contiguous()
    g = ops.tc_scan_backward(q, q.clone(), q.clone(), f32_dev(x["lam"]), f32_dev(x["eta"]), 8,
                             q.clone())
    torch.cuda.synchronize()
    assert g[0].shape == (1, 2, 0, d)
    assert torch.all(g[3] == 0) and torch.all(g[4] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_scan_backward_repeat_is_deterministic(d):
    x = I.draw(1, 2, 700, d, seed=9, dtype="f32")
    dm = I.draw_cotangent(1, 2, 700, d, seed=9)
    a = run(x, 64, dm)
    b = run(x, 64, dm)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_scan_backward_prefill_full_size_sampled_heads():
    # B=4 H=8 T=4096 d=64 W=512: the oracle on two whole heads (every b, t)
    w = I.WORKLOADS["prefill_scan_f32"]
    print("[case] scan backward prefill full size", flush=True)
    x = I.draw_workload("prefill_scan_f32")
    dm = I.draw_cotangent(w.B, w.H, w.T, w.d, seed=w.seed)
    got = run(x, w.W, dm)
    for h in (0, 5):
        sl = slice(h, h + 1)
        ref = O.tc_scan_backward(x["q64"][:, sl], x["k64"][:, sl], x["v64"][:, sl],
                                 x["lam"][sl].astype(np.float64), x["eta"][sl].astype(np.float64),
                                 w.W, dm[:, sl].astype(np.float64))
        for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta"), got, ref):
            check(f"head {h} {name}", a[:, sl] if a.ndim == 4 else a[sl], b, TOL)


@pytest.mark.parametrize("B,H,T,d,W", [(2, 3, 300, 32, 17), (1, 2, 1000, 64, 100), (1, 1, 20, 16, 45),
                                       (1, 3, 400, 128, 50)])
def test_scan_backward_through_the_gate(B, H, T, d, W):
    print(f"[case] gated scan backward B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=4500 + T, dtype="f32")
    dy = I.draw_cotangent(B, H, T, d, seed=4500 + T)
    g = np.linspace(-2.0, 1.5, H).astype(np.float32)
    out = ops.tc_scan_backward(to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
                               f32_dev(x["lam"]), f32_dev(x["eta"]), W, f32_dev(dy), g=f32_dev(g))
    torch.cuda.synchronize()
    ref = O.tc_gated_read_backward(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64),
                                   x["eta"].astype(np.float64), g.astype(np.float64), W, dy.astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta", "dg"), out, ref):
        check(f"gated {name}", a.cpu().numpy(), b, TOL)


@pytest.mark.parametrize("B,H,T,d,W", [(2, 3, 300, 32, 17), (1, 2, 1000, 64, 100), (1, 1, 256, 16, 32),
                                       (1, 2, 400, 128, 70)])
def test_scan_backward_bf16_inputs(B, H, T, d, W):
    # bf16 q, k, v are widened to fp32 in the workspace for dq, dlam and deta
    # (and, at d in {16, 32}, for dk and dv): those are the gradients of the bf16
    # values, near 1e-6 (dlam, a per-head sum with much cancellation when lam is
    # near 1, has reached 2e-5).  At d in {64, 128} dk and dv come from bf16
    # reads of the time-reversed sequences (about 2e-3).  Held to the bar for
    # bf16 inputs (2e-2).
    print(f"[case] scan backward bf16 B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=4300 + T + d, dtype="bf16")
    dm = I.draw_cotangent(B, H, T, d, seed=4300 + T + d)
    got = ops.tc_scan_backward(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), f32_dev(x["lam"]),
                               f32_dev(x["eta"]), W, f32_dev(dm))
    torch.cuda.synchronize()
    ref = O.tc_scan_backward(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64),
                             x["eta"].astype(np.float64), W, dm.astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta"), got, ref):
        check(f"bf16 {name}", a.cpu().numpy(), b, TOL_BF16)


@pytest.mark.parametrize("B,H,T,d,W,gated", [
    (1, 2, 1, 64, 4, False),      # one position, no eviction
    (1, 1, 50, 128, 64, False),   # T < W: every gradient 0
    (2, 2, 64, 64, 64, False),    # T = W
    (1, 3, 600, 64, 1, False),    # W = 1, several 256-row tiles
    (1, 2, 777, 128, 300, False),  # ragged last tile, evictions across tiles
    (2, 1, 513, 128, 32, True),   # through the gate
    (1, 2, 1100, 64, 257, True),
])
def test_scan_backward_bf16_reverse_reads(B, H, T, d, W, gated):
    # bf16 inputs with d in {64, 128}: dk and dv come from two bf16 forward
    # reads of the time-reversed sequences (cotangent scaled by the gate and
    # rounded to bf16 on the way), the rest from the fp32 kernels.
    print(f"[case] scan backward bf16 reversed reads B={B} H={H} T={T} d={d} W={W} gated={gated}", flush=True)
    x = I.draw(B, H, T, d, seed=4700 + T + d + W, dtype="bf16")
    dm = I.draw_cotangent(B, H, T, d, seed=4700 + T + d + W)
    args = [to_dev(x[n], "bf16") for n in ("q", "k", "v")] + [f32_dev(x["lam"]), f32_dev(x["eta"]), W,
                                                                f32_dev(dm)]
    lam64, eta64 = x["lam"].astype(np.float64), x["eta"].astype(np.float64)
    if gated:
        g = np.linspace(-1.5, 2.0, H).astype(np.float32)
        got = ops.tc_scan_backward(*args, g=f32_dev(g))
        ref = O.tc_gated_read_backward(x["q64"], x["k64"], x["v64"], lam64, eta64, g.astype(np.float64), W,
                                       dm.astype(np.float64))
        names = ("dq", "dk", "dv", "dlam", "deta", "dg")
    else:
        got = ops.tc_scan_backward(*args)
        ref = O.tc_scan_backward(x["q64"], x["k64"], x["v64"], lam64, eta64, W, dm.astype(np.float64))
        names = ("dq", "dk", "dv", "dlam", "deta")
    torch.cuda.synchronize()
    for name, a, b in zip(names, got, ref):
        a = a.cpu().numpy()
        if not np.any(b):
            assert not np.any(a), f"{name}: expected all zeros"
            continue
        check(f"bf16 reversed {name}", a, b, TOL_BF16)
    # rows with no pair: dk, dv rows i >= T - W are exactly 0
    z0 = max(T - W, 0)
    assert not np.any(got[1].cpu().numpy()[:, :, z0:]) and not np.any(got[2].cpu().numpy()[:, :, z0:])
