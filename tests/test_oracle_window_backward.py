"""Pins of the oracle's window-softmax backward and of the fused layer's
backward ("Tensor Cache: Eviction-conditioned Associative Memory for
Transformers", Methodology 1: the L1 cache's exact softmax and the gated
fusion y = y_local + sigmoid(g) m).  The pages give no backward; these pin
the reverse-mode functions against central differences of the forward
oracle, against torch autograd of an independently written band-masked
attention, and against closed forms.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

from oracle import tc as O


def rand(seed, B=1, H=2, T=11, d=3):
    rng = np.random.default_rng(seed)
    q, k, v, dy = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    lam = rng.uniform(0.5, 1.0, H)
    eta = rng.uniform(0.1, 1.0, H)
    g = rng.standard_normal(H)
    return q, k, v, dy, lam, eta, g


def fd(f, x, idx, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("W", [1, 3, 20])
def test_window_backward_matches_central_differences(W):
    q, k, v, dy, *_ = rand(1)
    scale = 0.7
    gq, gk, gv = O.window_softmax_backward(q, k, v, W, scale, dy)

    def loss(q_=q, k_=k, v_=v):
        return float(np.sum(O.window_softmax(q_, k_, v_, W, scale) * dy))

    for name, x, gx in (("q", q, gq), ("k", k, gk), ("v", v, gv)):
        for idx in [(0, 0, 0, 0), (0, 1, 5, 2), (0, 0, 10, 1), (0, 1, 7, 0)]:
            f = {"q": lambda z: loss(q_=z), "k": lambda z: loss(k_=z), "v": lambda z: loss(v_=z)}[name]
            assert abs(gx[idx] - fd(f, x, idx)) < 1e-8, (name, idx)


@pytest.mark.parametrize("W", [1, 4, 100])
def test_window_backward_matches_autograd_of_band_masked_attention(W):
    # written independently: the whole score matrix at once, a band mask
    # (j <= t and j > t - W), torch softmax, float64 autograd
    q, k, v, dy, *_ = rand(2, B=2, H=2, T=9, d=4)
    scale = 1.0 / math.sqrt(4)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    T = q.shape[2]
    t = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= t) & (j > t - W)
    s = torch.einsum("bhtd,bhjd->bhtj", tq, tk) * scale
    s = s.masked_fill(~mask, float("-inf"))
    y = torch.einsum("bhtj,bhjd->bhtd", torch.softmax(s, dim=-1), tv)
    (y * torch.tensor(dy)).sum().backward()
    gq, gk, gv = O.window_softmax_backward(q, k, v, W, scale, dy)
    np.testing.assert_allclose(gq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gv, tv.grad.numpy(), atol=1e-12)


def test_window_backward_one_token_window_is_the_identity():
    # W = 1: y = v, so dv = dy and q, k get nothing
    q, k, v, dy, *_ = rand(3)
    gq, gk, gv = O.window_softmax_backward(q, k, v, 1, 0.5, dy)
    assert np.all(gq == 0) and np.all(gk == 0)
    np.testing.assert_array_equal(gv, dy)


@pytest.mark.parametrize("W", [2, 5])
def test_fused_backward_matches_central_differences(W):
    q, k, v, dy, lam, eta, g = rand(4, T=10)
    gq, gk, gv, glam, geta, gg = O.tc_fused_backward(q, k, v, lam, eta, g, W, dy)

    def loss(q_=q, k_=k, v_=v, lam_=lam, eta_=eta, g_=g):
        return float(np.sum(O.tc_fused(q_, k_, v_, lam_, eta_, g_, W)[0] * dy))

    for name, x, gx in (("q", q, gq), ("k", k, gk), ("v", v, gv)):
        for idx in [(0, 0, 0, 0), (0, 1, 4, 2), (0, 0, 9, 1)]:
            f = {"q": lambda z: loss(q_=z), "k": lambda z: loss(k_=z), "v": lambda z: loss(v_=z)}[name]
            assert abs(gx[idx] - fd(f, x, idx)) < 1e-7, (name, idx)
    for name, x, gx in (("lam", lam, glam), ("eta", eta, geta), ("g", g, gg)):
        for idx in [(0,), (1,)]:
            f = {"lam": lambda z: loss(lam_=z), "eta": lambda z: loss(eta_=z), "g": lambda z: loss(g_=z)}[name]
            assert abs(gx[idx] - fd(f, x, idx)) < 1e-7, (name, idx)


def _window_mutant(kind):
    def run(q, k, v, W, scale, dy):
        gq, gk, gv = O.window_softmax_backward(q, k, v, W, scale, dy)
        if kind == "ds_without_the_mean_term":
            # the softmax Jacobian's -p p^T part dropped, in dq only
            gq2 = np.zeros_like(gq)
            T = q.shape[2]
            for t in range(T):
                lo = max(0, t - W + 1)
                s = np.einsum("bhjd,bhd->bhj", k[:, :, lo:t + 1], q[:, :, t]) * scale
                p = np.exp(s - s.max(-1, keepdims=True))
                p /= p.sum(-1, keepdims=True)
                dp = np.einsum("bhjd,bhd->bhj", v[:, :, lo:t + 1], dy[:, :, t])
                gq2[:, :, t] = scale * np.einsum("bhj,bhjd->bhd", p * dp, k[:, :, lo:t + 1])
            gq = gq2
        elif kind == "dk_one_token_late":
            gk = np.roll(gk, 1, axis=2)
        elif kind == "scale_missing":
            gq = gq / scale
        return gq, gk, gv
    return run


@pytest.mark.parametrize("kind", ["ds_without_the_mean_term", "dk_one_token_late", "scale_missing"])
def test_window_backward_pins_catch_planted_mistakes(kind):
    q, k, v, dy, *_ = rand(5)
    W, scale = 4, 0.7
    gq, gk, gv = _window_mutant(kind)(q, k, v, W, scale, dy)

    def loss(q_=q, k_=k):
        return float(np.sum(O.window_softmax(q_, k_, v, W, scale) * dy))

    worst = 0.0
    for idx in [(0, 0, 3, 0), (0, 1, 6, 2), (0, 0, 9, 1)]:
        worst = max(worst, abs(gq[idx] - fd(lambda z: loss(q_=z), q, idx)))
        worst = max(worst, abs(gk[idx] - fd(lambda z: loss(k_=z), k, idx)))
    assert worst > 1e-4
