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
