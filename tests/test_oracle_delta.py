"""Pins of the delta-rule oracle.

Page: "DeltaNet-family linear attention variants" (molayo1419.me): the
additive-write problem, DeltaNet's prediction-error write, locality in key
space and the reconstruction-loss derivation.  CPU only.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import delta as D

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(seed, B=2, H=2, T=30, dk=6, dv=5, beta_kind="u"):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    if beta_kind == "u":
        beta = rng.uniform(0, 1, (B, H, T))
    elif beta_kind == "1":
        beta = np.ones((B, H, T))
    else:
        beta = np.zeros((B, H, T))
    return q, k, v, beta


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def test_hand_example():
    with open(os.path.join(GOLD, "delta_hand_example.json")) as f:
        g = json.load(f)
    i = g["inputs"]
    q, k, v = (np.array(i[n], float)[None, None] for n in ("q", "k", "v"))
    beta = np.array(i["beta"], float)[None, None]
    o, S = D.delta_scan(q, k, v, beta)
    np.testing.assert_allclose(o[0, 0], g["o"], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], g["S_final"], atol=1e-12)


def _states(q, k, v, beta):
    """All intermediate states S_0..S_T, by running the oracle on prefixes."""
    T = q.shape[2]
    out = [np.zeros(q.shape[:2] + (v.shape[-1], q.shape[-1]))]
    for t in range(1, T + 1):
        out.append(D.delta_scan(q[:, :, :t], k[:, :, :t], v[:, :, :t], beta[:, :, :t])[1])
    return out


def test_beta_one_rereads_value_exactly():
    # beta = 1: reading the just-written key returns exactly v_t (normalised keys).
    q, k, v, beta = rand_inputs(1, beta_kind="1")
    S = _states(q, k, v, beta)
    for t in range(q.shape[2]):
        rd = np.einsum("bhij,bhj->bhi", S[t + 1], k[:, :, t])
        np.testing.assert_allclose(rd, v[:, :, t], rtol=0, atol=1e-12)


def test_general_reread_interpolates():
    # Immediate re-read gives (1 - beta) S_{t-1} k_t + beta v_t.
    q, k, v, beta = rand_inputs(2)
    S = _states(q, k, v, beta)
    for t in range(q.shape[2]):
        rd = np.einsum("bhij,bhj->bhi", S[t + 1], k[:, :, t])
        prev = np.einsum("bhij,bhj->bhi", S[t], k[:, :, t])
        b = beta[:, :, t, None]
        np.testing.assert_allclose(rd, (1 - b) * prev + b * v[:, :, t], rtol=1e-12, atol=1e-12)


def test_orthogonal_query_unchanged():
    # The update is local in key space: a query orthogonal to k_t sees no change.
    q, k, v, beta = rand_inputs(3)
    S = _states(q, k, v, beta)
    rng = np.random.default_rng(0)
    for t in range(q.shape[2]):
        x = rng.standard_normal(k.shape[:2] + (k.shape[-1],))
        kt = k[:, :, t]
        x -= np.einsum("bhd,bhd->bh", x, kt)[..., None] * kt  # project out k_t
        before = np.einsum("bhij,bhj->bhi", S[t], x)
        after = np.einsum("bhij,bhj->bhi", S[t + 1], x)
        np.testing.assert_allclose(after, before, rtol=0, atol=1e-12)


def test_update_is_gradient_step_on_reconstruction_loss():
    # S_t = S_{t-1} - beta_t * grad_S 1/2 ||S k_t - v_t||^2 at S_{t-1}; the gradient is
    # taken by central finite differences (independent of the closed form).
    q, k, v, beta = rand_inputs(4, B=1, H=1, T=6, dk=3, dv=2)
    S = _states(q, k, v, beta)
    h = 1e-6
    for t in range(q.shape[2]):
        Sp = S[t][0, 0]
        grad = np.zeros_like(Sp)
        for i in range(Sp.shape[0]):
            for j in range(Sp.shape[1]):
                e = np.zeros_like(Sp)
                e[i, j] = h
                grad[i, j] = (D.reconstruction_loss(Sp + e, k[0, 0, t], v[0, 0, t])
                              - D.reconstruction_loss(Sp - e, k[0, 0, t], v[0, 0, t])) / (2 * h)
        np.testing.assert_allclose(S[t + 1][0, 0], Sp - beta[0, 0, t] * grad, rtol=0, atol=1e-8)


def test_beta_zero_reads_zero():
    q, k, v, beta = rand_inputs(5, beta_kind="0")
    o, S = D.delta_scan(q, k, v, beta)
    assert np.all(o == 0) and np.all(S == 0)


def test_repeated_key_replaces_while_additive_accumulates():
    # Additive-write problem: writing v1 then v2 under the same normalised key returns
    # v1 + v2 for linear attention, but v2 for the delta rule with beta = 1.
    rng = np.random.default_rng(6)
    kk = rng.standard_normal(4)
    kk /= np.linalg.norm(kk)
    k = np.stack([kk, kk])[None, None]
    v = rng.standard_normal((1, 1, 2, 3))
    q = k.copy()
    od, _ = D.delta_scan(q, k, v, np.ones((1, 1, 2)))
    oa, _ = D.additive_scan(q, k, v)
    np.testing.assert_allclose(od[0, 0, 1], v[0, 0, 1], atol=1e-12)
    np.testing.assert_allclose(oa[0, 0, 1], v[0, 0, 0] + v[0, 0, 1], atol=1e-12)


def test_additive_scan_is_unnormalised_causal_linear_attention():
    q, k, v, _ = rand_inputs(7)
    o, _ = D.additive_scan(q, k, v)
    T = q.shape[2]
    s = np.einsum("bhtd,bhjd->bhtj", q, k) * np.tril(np.ones((T, T)))
    np.testing.assert_allclose(o, np.einsum("bhtj,bhje->bhte", s, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,C", [(130, 64), (64, 64), (7, 64), (45, 8), (1, 4)])
@pytest.mark.parametrize("beta_kind", ["u", "1", "0"])
def test_chunked_equals_sequential(T, C, beta_kind):
    q, k, v, beta = rand_inputs(8, T=T, beta_kind=beta_kind)
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal(q.shape[:2] + (v.shape[-1], q.shape[-1])) * 0.3
    o, S = D.delta_scan(q, k, v, beta, S0)
    oc, Sc = D.delta_scan_chunked(q, k, v, beta, C, S0)
    assert np.max(np.abs(oc - o)) <= 1e-12 * max(1, np.max(np.abs(o)))
    assert np.max(np.abs(Sc - S)) <= 1e-12 * max(1, np.max(np.abs(S)))


@settings(max_examples=30, deadline=None)
@given(T=st.integers(1, 30), C=st.integers(1, 9), d=st.integers(1, 5), seed=st.integers(0, 9999))
def test_property_chunked_equals_sequential(T, C, d, seed):
    q, k, v, beta = rand_inputs(seed, B=1, H=1, T=T, dk=d, dv=d)
    o, S = D.delta_scan(q, k, v, beta)
    oc, Sc = D.delta_scan_chunked(q, k, v, beta, C)
    assert np.max(np.abs(oc - o)) <= 1e-10 * max(1, np.max(np.abs(o)))


def _mutant_read_before_write(q, k, v, beta):
    B, H, T, dk = q.shape
    S = np.zeros((B, H, v.shape[-1], dk))
    o = np.zeros((B, H, T, v.shape[-1]))
    for t in range(T):
        o[:, :, t] = np.einsum("bhij,bhj->bhi", S, q[:, :, t])
        e = beta[:, :, t, None] * (v[:, :, t] - np.einsum("bhij,bhj->bhi", S, k[:, :, t]))
        S = S + e[..., :, None] * k[:, :, t, None, :]
    return o, S


def _mutant_sign(q, k, v, beta):
    return D.delta_scan(q, k, -v, beta)


@pytest.mark.parametrize("mutant", [_mutant_read_before_write, _mutant_sign])
def test_hand_example_catches_planted_mistakes(mutant):
    with open(os.path.join(GOLD, "delta_hand_example.json")) as f:
        g = json.load(f)
    i = g["inputs"]
    q, k, v = (np.array(i[n], float)[None, None] for n in ("q", "k", "v"))
    o, _ = mutant(q, k, v, np.array(i["beta"], float)[None, None])
    assert np.max(np.abs(o[0, 0] - np.array(g["o"]))) > 1e-6


# ---------------------------------------------------------------- backward

def _delta_loss(q, k, v, beta, do, S0=None, dSf=None):
    o, S = D.delta_scan(q, k, v, beta, S0)
    out = float(np.sum(o * do))
    if dSf is not None:
        out += float(np.sum(S * dSf))
    return out


@pytest.mark.parametrize("with_state", [False, True])
def test_delta_backward_matches_central_differences(with_state):
    q, k, v, beta = rand_inputs(70, B=1, H=2, T=9, dk=3, dv=4)
    rng = np.random.default_rng(71)
    do = rng.standard_normal(v.shape)
    S0 = rng.standard_normal((1, 2, 4, 3)) if with_state else None
    dSf = rng.standard_normal((1, 2, 4, 3)) if with_state else None
    gq, gk, gv, gb, gS0 = D.delta_scan_backward(q, k, v, beta, do, S0, dSf)
    h = 1e-6
    args = {"q": q, "k": k, "v": v, "beta": beta}
    grads = {"q": gq, "k": gk, "v": gv, "beta": gb}
    for name, x in args.items():
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            a = dict(args)
            a[name] = x.copy()
            a[name][i] += h
            lp = _delta_loss(a["q"], a["k"], a["v"], a["beta"], do, S0, dSf)
            a[name][i] -= 2 * h
            lm = _delta_loss(a["q"], a["k"], a["v"], a["beta"], do, S0, dSf)
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)
    if with_state:
        fd = np.zeros_like(S0)
        it = np.nditer(S0, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            sp, sm = S0.copy(), S0.copy()
            sp[i] += h
            sm[i] -= h
            fd[i] = (_delta_loss(q, k, v, beta, do, sp, dSf) - _delta_loss(q, k, v, beta, do, sm, dSf)) / (2 * h)
        np.testing.assert_allclose(gS0, fd, rtol=1e-6, atol=1e-8)


def test_delta_backward_matches_autograd_of_the_per_token_rule():
    torch = pytest.importorskip("torch")
    q, k, v, beta = rand_inputs(72, B=2, H=1, T=20, dk=4, dv=3)
    do = np.random.default_rng(73).standard_normal(v.shape)
    gq, gk, gv, gb, _ = D.delta_scan_backward(q, k, v, beta, do)
    tq, tk, tv, tb = (torch.tensor(a, requires_grad=True) for a in (q, k, v, beta))
    # the rule written as S_t = S_{t-1} (I - beta k k^T) + beta v k^T
    S = torch.zeros(2, 1, 3, 4, dtype=torch.float64)
    outs = []
    eye = torch.eye(4, dtype=torch.float64)
    for t in range(20):
        kt, bt = tk[:, :, t], tb[:, :, t, None, None]
        S = S @ (eye - bt * kt[..., :, None] * kt[..., None, :]) + bt * tv[:, :, t, :, None] * kt[..., None, :]
        outs.append(S @ tq[:, :, t, :, None])
    o = torch.cat(outs, dim=-1).transpose(-1, -2)
    (o * torch.tensor(do)).sum().backward()
    for a, b in ((gq, tq), (gk, tk), (gv, tv), (gb, tb)):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_delta_backward_beta_zero_special_case():
    # beta = 0: nothing is written, o_t = S0 q_t; dq = S0^T do, dk = dv = 0,
    # dbeta_t = <(sum_{s>=t} do_s q_s^T) k_t, v_t - S0 k_t>
    q, k, v, _ = rand_inputs(74, B=1, H=1, T=7, dk=3, dv=2)
    rng = np.random.default_rng(75)
    do = rng.standard_normal(v.shape)
    S0 = rng.standard_normal((1, 1, 2, 3))
    gq, gk, gv, gb, gS0 = D.delta_scan_backward(q, k, v, np.zeros((1, 1, 7)), do, S0)
    np.testing.assert_allclose(gq[0, 0], do[0, 0] @ S0[0, 0], rtol=1e-13)
    assert np.all(gk == 0) and np.all(gv == 0)
    for t in range(7):
        G = sum(np.outer(do[0, 0, s], q[0, 0, s]) for s in range(t, 7))
        want = (G @ k[0, 0, t]) @ (v[0, 0, t] - S0[0, 0] @ k[0, 0, t])
        assert abs(gb[0, 0, t] - want) < 1e-12
    np.testing.assert_allclose(gS0[0, 0], sum(np.outer(do[0, 0, s], q[0, 0, s]) for s in range(7)), rtol=1e-13)


def _delta_backward_mutant(q, k, v, beta, do, kind):
    # the reverse sweep of the oracle with one planted mistake
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk))
    states = [S.copy()]
    for t in range(T):
        e = beta[:, :, t, None] * (v[:, :, t] - np.einsum("bhij,bhj->bhi", S, k[:, :, t]))
        S = S + e[..., :, None] * k[:, :, t, None, :]
        states.append(S.copy())
    gq, gk, gb = np.zeros_like(q), np.zeros_like(k), np.zeros_like(beta)
    dS = np.zeros((B, H, dv, dk))
    for t in range(T - 1, -1, -1):
        S_t, S_prev = states[t + 1], states[t]
        dS = dS + do[:, :, t, :, None] * q[:, :, t, None, :]
        gq[:, :, t] = np.einsum("bhij,bhi->bhj", S_t, do[:, :, t])
        resid = v[:, :, t] - np.einsum("bhij,bhj->bhi", S_prev, k[:, :, t])
        e = beta[:, :, t, None] * resid
        de = np.einsum("bhij,bhj->bhi", dS, k[:, :, t])
        gb[:, :, t] = np.einsum("bhi,bhi->bh", de, resid) * (-1.0 if kind == "dbeta_sign" else 1.0)
        gk[:, :, t] = np.einsum("bhij,bhi->bhj", dS, e)
        if kind != "dk_missing_read_term":
            gk[:, :, t] -= beta[:, :, t, None] * np.einsum("bhij,bhi->bhj", S_prev, de)
        if kind != "dS_no_erase":
            dS = dS - beta[:, :, t, None, None] * de[..., :, None] * k[:, :, t, None, :]
    return gq, gk, gb


@pytest.mark.parametrize("kind", ["dk_missing_read_term", "dbeta_sign", "dS_no_erase", "none"])
def test_delta_backward_pins_catch_planted_mistakes(kind):
    q, k, v, beta = rand_inputs(76, B=1, H=1, T=6, dk=2, dv=2)
    do = np.random.default_rng(77).standard_normal(v.shape)
    gq, gk, gb = _delta_backward_mutant(q, k, v, beta, do, kind)
    h = 1e-6
    worst = 0.0
    for name, x, g in (("k", k, gk), ("beta", beta, gb)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"k": k, "beta": beta}
            a[name] = xp
            lp = _delta_loss(q, a["k"], v, a["beta"], do)
            a[name] = xm
            lm = _delta_loss(q, a["k"], v, a["beta"], do)
            worst = max(worst, abs(g[idx] - (lp - lm) / (2 * h)))
    if kind == "none":
        assert worst < 1e-7  # the unmutated sweep passes the same check
    else:
        assert worst > 1e-4
