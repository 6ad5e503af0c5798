"""Parity of tc_scan_backward (C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, report, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5


def run(x, W, dm):
    g = ops.tc_scan_backward(to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
                             f32_dev(x["lam"]), f32_dev(x["eta"]), W, f32_dev(dm))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in g]


def check(x, W, dm, label):
    got = run(x, W, dm)
    ref = O.tc_scan_backward(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64),
                             x["eta"].astype(np.float64), W, dm.astype(np.float64))
    for name, a, b in zip(("dq", "dk", "dv", "dlam", "deta"), got, ref):
        assert report(f"{label} {name}", a, b) <= TOL, name
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
])
def test_scan_backward_small(B, H, T, d, W):
    print(f"[case] scan backward B={B} H={H} T={T} d={d} W={W}", flush=True)
    x = I.draw(B, H, T, d, seed=4000 + T + d, dtype="f32")
    dm = I.draw_cotangent(B, H, T, d, seed=4000 + T + d)
    check(x, W, dm, "small")


@pytest.mark.parametrize("lam_val", [0.0, 1.0, 0.5])
def test_scan_backward_lambda_edges(lam_val):
    print(f"[case] scan backward lam={lam_val}", flush=True)
    x = I.draw(2, 2, 333, 64, seed=78, dtype="f32", lam=("fixed", lam_val))
    dm = I.draw_cotangent(2, 2, 333, 64, seed=78)
    check(x, 20, dm, f"lam={lam_val}")


def test_scan_backward_empty_sequence():
    x = I.draw(1, 2, 1, 64, seed=5, dtype="f32")
    q = to_dev(x["q"], "f32")[:, :, :0].contiguous()
    g = ops.tc_scan_backward(q, q.clone(), q.clone(), f32_dev(x["lam"]), f32_dev(x["eta"]), 8,
                             q.clone())
    torch.cuda.synchronize()
    assert g[0].shape == (1, 2, 0, 64)
    assert torch.all(g[3] == 0) and torch.all(g[4] == 0)


def test_scan_backward_repeat_is_deterministic():
    x = I.draw(1, 2, 700, 64, seed=9, dtype="f32")
    dm = I.draw_cotangent(1, 2, 700, 64, seed=9)
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
            assert report(f"head {h} {name}", a[:, sl] if a.ndim == 4 else a[sl], b) <= TOL, name


@pytest.mark.parametrize("B,H,T,d,W", [(2, 3, 300, 32, 17), (1, 2, 1000, 64, 100), (1, 1, 20, 16, 45)])
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
        assert report(f"gated {name}", a.cpu().numpy(), b) <= TOL, name
