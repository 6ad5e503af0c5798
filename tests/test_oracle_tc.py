"""Pins of the Tensor Cache oracle against things other than itself.

Page: "Tensor Cache: Eviction-conditioned Associative Memory for Transformers"
(Methodology 1 and 2, Main contributions), with the linear-attention identity
of the DeltaNet-variants page and the Hebbian memory of the Hebbian-MLP page.
Every check here is CPU-only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import tc as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(seed, B=2, H=2, T=40, dk=5, dv=4, unit_keys=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    lam = rng.uniform(0.5, 1.0, H)
    eta = rng.uniform(0.1, 1.0, H)
    g = rng.standard_normal(H)
    return q, k, v, lam, eta, g


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def brute_force_m(q, k, v, lam, eta, W):
    """Pure-Python double sum m_t = sum_{i<=t-W} eta lam^((t-W)-i) <q_t,k_i> v_i."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                for i in range(0, t - W + 1):
                    w = eta[h] * lam[h] ** ((t - W) - i)
                    dot = sum(q[b, h, t, a] * k[b, h, i, a] for a in range(dk))
                    for c in range(dv):
                        out[b, h, t, c] += w * dot * v[b, h, i, c]
    return out


# ---------------------------------------------------------------- hand examples

def test_hand_examples():
    with open(os.path.join(GOLD, "tc_hand_examples.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    q = np.array(inp["q"], float)[None, None]
    k = np.array(inp["k"], float)[None, None]
    v = np.array(inp["v"], float)[None, None]
    lam = np.array([inp["lam"]])
    eta = np.array([inp["eta"]])
    for case in g["cases"]:
        W = case["W"]
        m, A = O.tc_scan(q, k, v, lam, eta, W)
        np.testing.assert_allclose(m[0, 0], case["m"], atol=1e-12)
        np.testing.assert_allclose(A[0, 0], case["A_final"], atol=1e-12)
        y, _ = O.tc_fused(q, k, v, lam, eta, np.array([case["g"]]), W, scale=case["scale"])
        np.testing.assert_allclose(y[0, 0], case["y"], atol=1e-12)


# ---------------------------------------------------------------- L2 memory

@pytest.mark.parametrize("W", [1, 3, 7, 40, 45])
@pytest.mark.parametrize("lam_kind", ["rand", "zero", "one"])
def test_brute_force_double_sum(W, lam_kind):
    q, k, v, lam, eta, _ = rand_inputs(1 + W, B=1, H=2, T=24, dk=3, dv=2)
    if lam_kind == "zero":
        lam = np.zeros_like(lam)
    elif lam_kind == "one":
        lam = np.ones_like(lam)
    m, _ = O.tc_scan(q, k, v, lam, eta, W)
    ref = brute_force_m(q, k, v, lam, eta, W)
    assert np.max(np.abs(m - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_lambda_one_is_cumulative_hebbian_sum():
    # lam = 1: A_t = eta * sum_{i <= t-W} k_i v_i^T, the classical Hebbian memory
    # W = sum v k^T of the Hebbian-MLP page (transposed orientation), via np.cumsum.
    q, k, v, lam, eta, _ = rand_inputs(2, T=50)
    lam = np.ones_like(lam)
    W = 6
    m, A = O.tc_scan(q, k, v, lam, eta, W)
    outer = k[..., :, None] * v[..., None, :]  # [B,H,T,dk,dv]
    cums = np.cumsum(outer, axis=2)
    T = q.shape[2]
    ref = np.zeros_like(m)
    for t in range(W, T):
        ref[:, :, t] = eta[None, :, None] * np.einsum("bhd,bhde->bhe", q[:, :, t], cums[:, :, t - W])
    np.testing.assert_allclose(m, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A, eta[None, :, None, None] * cums[:, :, T - 1 - W], rtol=1e-12, atol=1e-13)


def test_lambda_zero_keeps_only_last_eviction():
    q, k, v, lam, eta, _ = rand_inputs(3, T=30)
    W = 4
    m, _ = O.tc_scan(q, k, v, np.zeros_like(lam), eta, W)
    ref = np.zeros_like(m)
    for t in range(W, q.shape[2]):
        dot = np.einsum("bhd,bhd->bh", q[:, :, t], k[:, :, t - W])
        ref[:, :, t] = eta[None, :, None] * dot[..., None] * v[:, :, t - W]
    np.testing.assert_allclose(m, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("W", [30, 31, 100])
def test_window_covering_sequence_reads_zero(W):
    q, k, v, lam, eta, _ = rand_inputs(4, T=30)
    m, A = O.tc_scan(q, k, v, lam, eta, W)
    assert np.all(m == 0.0) and np.all(A == 0.0)


def test_single_write_is_linear_attention_identity():
    # One eviction: q (k (x) v) = <q, k> v (read identity of the Tensor Cache page,
    # core identity of the DeltaNet-variants page).
    q, k, v, lam, eta, _ = rand_inputs(5, T=9)
    W = 8
    m, A = O.tc_scan(q, k, v, lam, eta, W)
    dot = np.einsum("bhd,bhd->bh", q[:, :, 8], k[:, :, 0])
    np.testing.assert_allclose(m[:, :, 8], eta[None, :, None] * dot[..., None] * v[:, :, 0], rtol=1e-13)
    assert np.all(m[:, :, :8] == 0.0)


def test_partition_identity_each_token_counted_once():
    # Main contributions: tokens split cleanly into L1-resident and L2-compressed.
    # With lam = eta = 1, the L2 read plus the plain linear sum over the L1 window
    # equals causal linear attention over all tokens (computed as one masked product).
    q, k, v, lam, eta, _ = rand_inputs(6, T=37)
    ones = np.ones_like(lam)
    for W in (1, 5, 16, 37, 50):
        m, _ = O.tc_scan(q, k, v, ones, ones, W)
        T = q.shape[2]
        s = np.einsum("bhtd,bhjd->bhtj", q, k)
        causal = np.tril(np.ones((T, T)))
        full = np.einsum("bhtj,bhje->bhte", s * causal, v)
        rel_win = np.tril(np.ones((T, T))) - np.tril(np.ones((T, T)), -W)
        local = np.einsum("bhtj,bhje->bhte", s * rel_win, v)
        np.testing.assert_allclose(m + local, full, rtol=1e-11, atol=1e-12)


def test_closed_form_rows_match_recurrence():
    q, k, v, lam, eta, _ = rand_inputs(7, T=70)
    W = 9
    m, _ = O.tc_scan(q, k, v, lam, eta, W)
    rows = [0, 8, 9, 10, 33, 69]
    np.testing.assert_allclose(O.tc_scan_rows(q, k, v, lam, eta, W, rows), m[:, :, rows], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,W,C", [(200, 13, 64), (64 + 5, 5, 64), (257, 1, 64), (40, 3, 8), (50, 60, 64)])
def test_chunked_scan_equals_sequential(T, W, C):
    # Methodology 2: the parallel weighted-sum scan equals the sequential writes.
    q, k, v, lam, eta, _ = rand_inputs(8, T=T)
    for lam_v in (lam, np.zeros_like(lam), np.ones_like(lam)):
        m, A = O.tc_scan(q, k, v, lam_v, eta, W)
        mc, Ac = O.tc_scan_chunked(q, k, v, lam_v, eta, W, C)
        assert rel(mc, m) <= 1e-12
        assert rel(Ac, A) <= 1e-12


def test_chunk_mean_shortcut_is_wrong():
    # Methodology 2: the chunk-mean shortcut adds spurious cross products; it must
    # differ visibly from the sequential oracle on random data.
    q, k, v, lam, eta, _ = rand_inputs(9, T=300)
    m, _ = O.tc_scan(q, k, v, lam, eta, 20)
    mm, _ = O.chunk_mean_scan(q, k, v, lam, eta, 20, C=64)
    assert rel(mm, m) > 1e-3


def test_chunk_mean_cross_product_count():
    # With one-hot keys/values e_i, the true chunk write sum_i k_i v_i^T is the identity,
    # while C * mean(k) (x) mean(v) has C^2 - C nonzero off-diagonal entries.
    C = 8
    d = 8
    k = np.eye(d)[None, None, :C]
    v = np.eye(d)[None, None, :C]
    q = np.zeros_like(k)
    one = np.ones(1)
    _, A_true = O.tc_scan(q, np.concatenate([k, k[:, :, :1]], 2), np.concatenate([v, v[:, :, :1]], 2),
                          one, one, 1)
    _, A_mean = O.chunk_mean_scan(q, k, v, one, one, 0, C=C)
    off = ~np.eye(d, dtype=bool)
    assert np.count_nonzero(np.abs(A_true[0, 0][off]) > 1e-15) == 0
    assert np.count_nonzero(np.abs(A_mean[0, 0][off]) > 1e-15) == C * C - C


# ---------------------------------------------------------------- streaming ring

@pytest.mark.parametrize("W", [1, 4, 9])
def test_decoder_ring_matches_scan(W):
    q, k, v, lam, eta, _ = rand_inputs(10, T=30)
    m, A = O.tc_scan(q, k, v, lam, eta, W)
    B, H, T, dk = q.shape
    dec = O.TensorCacheDecoder(B, H, dk, v.shape[-1], W, lam, eta)
    for t in range(T):
        mt = dec.step(q[:, :, t], k[:, :, t], v[:, :, t])
        np.testing.assert_allclose(mt, m[:, :, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dec.A, A, rtol=1e-12, atol=1e-14)
    # the ring holds exactly the last W tokens at slots pos mod W
    for t in range(max(0, T - W), T):
        np.testing.assert_array_equal(dec.ring_k[:, :, t % W], k[:, :, t])


def test_scan_then_decode_equals_longer_scan():
    # Streaming continuation: prefill with the scan, hand over A_final and the last W
    # tokens as the ring, continue with single steps.
    q, k, v, lam, eta, _ = rand_inputs(11, T=45)
    W, T0 = 7, 30
    m_full, A_full = O.tc_scan(q, k, v, lam, eta, W)
    _, A0 = O.tc_scan(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], lam, eta, W)
    B, H = q.shape[:2]
    ring_k = np.zeros((B, H, W, q.shape[-1]))
    ring_v = np.zeros((B, H, W, v.shape[-1]))
    for t in range(T0 - W, T0):
        ring_k[:, :, t % W] = k[:, :, t]
        ring_v[:, :, t % W] = v[:, :, t]
    dec = O.TensorCacheDecoder.from_state(ring_k, ring_v, A0, np.full(B, T0), W, lam, eta)
    for t in range(T0, 45):
        np.testing.assert_allclose(dec.step(q[:, :, t], k[:, :, t], v[:, :, t]), m_full[:, :, t],
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dec.A, A_full, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- L1 and fusion

def test_window_covering_sequence_is_causal_softmax_attention():
    q, k, v, *_ = rand_inputs(12, T=33)
    scale = 1 / math.sqrt(q.shape[-1])
    y = O.window_softmax(q, k, v, 1000, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=scale).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_window_is_banded_softmax_attention():
    # sliding window = softmax attention under a band mask (library routine with an explicit mask)
    q, k, v, *_ = rand_inputs(13, T=40)
    W, scale = 6, 0.37
    T = q.shape[2]
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(band), scale=scale).numpy()
    np.testing.assert_allclose(O.window_softmax(q, k, v, W, scale), ref, rtol=1e-12, atol=1e-13)


def test_window_one_returns_value():
    q, k, v, *_ = rand_inputs(14, T=20)
    np.testing.assert_array_equal(O.window_softmax(q, k, v, 1, 0.5), v)


def test_gate_limits():
    q, k, v, lam, eta, _ = rand_inputs(15, T=30)
    W = 5
    scale = 0.4
    y_loc = O.window_softmax(q, k, v, W, scale)
    m, _ = O.tc_scan(q, k, v, lam, eta, W)
    y_off, _ = O.tc_fused(q, k, v, lam, eta, np.full(2, -1e4), W, scale)
    np.testing.assert_array_equal(y_off, y_loc)  # sigmoid(-inf) -> pure sliding window
    y_half, _ = O.tc_fused(q, k, v, lam, eta, np.zeros(2), W, scale)
    np.testing.assert_allclose(y_half, y_loc + 0.5 * m, rtol=1e-14, atol=1e-15)


def test_fused_rows_match_full():
    q, k, v, lam, eta, g = rand_inputs(16, T=50)
    W = 8
    y, _ = O.tc_fused(q, k, v, lam, eta, g, W)
    rows = [0, 7, 8, 9, 31, 49]
    np.testing.assert_allclose(O.tc_fused_rows(q, k, v, lam, eta, g, W, rows), y[:, :, rows],
                               rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- full decode step

def run_layer_decoder(q, k, v, lam, eta, g, W, scale):
    B, H, T, dk = q.shape
    dec = O.TensorCacheDecoder(B, H, dk, v.shape[-1], W, lam, eta)
    return np.stack([dec.step_layer(q[:, :, t], k[:, :, t], v[:, :, t], g, scale) for t in range(T)],
                    axis=2)


def test_decode_layer_without_evictions_is_causal_softmax_attention():
    # W >= T: nothing leaves the ring, A stays 0, and the L1 part is causal attention
    q, k, v, lam, eta, g = rand_inputs(40, T=25)
    scale = 0.6
    y = run_layer_decoder(q, k, v, lam, eta, g, 64, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=scale).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_decode_layer_l1_is_banded_softmax_attention():
    # eta = 0: the L2 read is 0, and the ring softmax is attention under the W-band mask
    q, k, v, lam, _, g = rand_inputs(41, T=40)
    W, scale = 7, 0.45
    T = q.shape[2]
    y = run_layer_decoder(q, k, v, lam, np.zeros(2), g, W, scale)
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(band), scale=scale).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_decode_layer_adds_gated_l2_read():
    # y(eta) - y(eta = 0) = sigmoid(g) m, m from the brute-force double sum
    q, k, v, lam, eta, g = rand_inputs(42, T=36)
    W, scale = 5, 0.3
    y1 = run_layer_decoder(q, k, v, lam, eta, g, W, scale)
    y0 = run_layer_decoder(q, k, v, lam, np.zeros(2), g, W, scale)
    m = brute_force_m(q, k, v, lam, eta, W)
    gate = 1.0 / (1.0 + np.exp(-g))
    np.testing.assert_allclose(y1 - y0, gate[None, :, None, None] * m, rtol=1e-11, atol=1e-13)


def test_decode_layer_equal_keys_average_the_window():
    # every key the same: every score the same, so the L1 output is the mean of the
    # values in the window (the W most recent, the current one included)
    q, k, v, lam, _, g = rand_inputs(43, T=30)
    k[...] = k[:, :, :1, :]
    W = 6
    y = run_layer_decoder(q, k, v, lam, np.zeros(2), g, W, 1.0)
    for t in range(q.shape[2]):
        np.testing.assert_allclose(y[:, :, t], v[:, :, max(0, t - W + 1): t + 1].mean(axis=2),
                                   rtol=1e-12, atol=1e-14)


def test_decode_layer_continues_a_prefill():
    # prefill with the fused layer's oracle, hand over A and the last W tokens as the
    # ring, continue with full decode steps: the rows equal the longer prefill
    q, k, v, lam, eta, g = rand_inputs(44, T=41)
    W, T0, scale = 6, 27, 0.5
    y_full, A_full = O.tc_fused(q, k, v, lam, eta, g, W, scale)
    _, A0 = O.tc_fused(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], lam, eta, g, W, scale)
    B, H = q.shape[:2]
    ring_k = np.zeros((B, H, W, q.shape[-1]))
    ring_v = np.zeros((B, H, W, v.shape[-1]))
    for t in range(T0 - W, T0):
        ring_k[:, :, t % W] = k[:, :, t]
        ring_v[:, :, t % W] = v[:, :, t]
    dec = O.TensorCacheDecoder.from_state(ring_k, ring_v, A0, np.full(B, T0), W, lam, eta)
    for t in range(T0, q.shape[2]):
        np.testing.assert_allclose(dec.step_layer(q[:, :, t], k[:, :, t], v[:, :, t], g, scale),
                                   y_full[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec.A, A_full, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- properties

@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 40), W=st.integers(1, 43), d=st.integers(1, 6),
       lam_kind=st.sampled_from(["u", "0", "1"]), seed=st.integers(0, 10_000))
def test_property_recurrence_equals_brute_force(T, W, d, lam_kind, seed):
    q, k, v, lam, eta, _ = rand_inputs(seed, B=1, H=1, T=T, dk=d, dv=max(1, d - 1))
    lam = {"u": lam, "0": np.zeros(1), "1": np.ones(1)}[lam_kind]
    m, _ = O.tc_scan(q, k, v, lam, eta, W)
    ref = brute_force_m(q, k, v, lam, eta, W)
    assert np.max(np.abs(m - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref)))
    mc, _ = O.tc_scan_chunked(q, k, v, lam, eta, W, C=4)
    assert np.max(np.abs(mc - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- planted mistakes

def _mutant_off_by_one(q, k, v, lam, eta, W):
    return O.tc_scan(q, k, v, lam, eta, W + 1)


def _mutant_read_before_write(q, k, v, lam, eta, W):
    qq = np.concatenate([q[:, :, 1:], q[:, :, :1]], axis=2)
    m, A = O.tc_scan(qq, k, v, lam, eta, W)
    out = np.zeros_like(m)
    out[:, :, 1:] = m[:, :, :-1]
    return out, A


def _mutant_transposed(q, k, v, lam, eta, W):
    return O.tc_scan(q, v, k, lam, eta, W)


def _mutant_no_decay(q, k, v, lam, eta, W):
    return O.tc_scan(q, k, v, np.ones_like(lam), eta, W)


@pytest.mark.parametrize("mutant", [_mutant_off_by_one, _mutant_read_before_write, _mutant_transposed,
                                    _mutant_no_decay])
def test_brute_force_pin_catches_planted_mistakes(mutant):
    # The brute-force pin must reject plausible slips (copies of the oracle with one
    # planted mistake each).
    q, k, v, lam, eta, _ = rand_inputs(17, B=1, H=2, T=20, dk=3, dv=3)
    ref = brute_force_m(q, k, v, lam, eta, 4)
    m, _ = mutant(q, k, v, lam, eta, 4)
    assert np.max(np.abs(m - ref)) > 1e-6


# Copies of the full decode step with one planted mistake each; the decode-layer pins
# above (banded attention, gated read) must reject every one.
def _layer_mutant(kind):
    def run(q, k, v, lam, eta, g, W, scale):
        B, H, T, _ = q.shape
        m = O.tc_scan(q, k, v, lam, eta, W)[0]
        gate = 1.0 / (1.0 + np.exp(-g))
        y = np.zeros(v.shape)
        for t in range(T):
            lo, hi = {"no_current": (t - W, t), "window_plus_one": (t - W, t + 1)}.get(kind, (t - W + 1, t + 1))
            lo = max(0, lo)
            yl = np.zeros((B, H, v.shape[-1]))
            if hi > lo:
                s = np.einsum("bhjd,bhd->bhj", k[:, :, lo:hi], q[:, :, t]) * scale
                p = np.exp(s - s.max(axis=-1, keepdims=True))
                p /= p.sum(axis=-1, keepdims=True)
                yl = np.einsum("bhj,bhjd->bhd", p, v[:, :, lo:hi])
            if kind == "gate_on_local":
                y[:, :, t] = gate[None, :, None] * yl + m[:, :, t]
            else:
                y[:, :, t] = yl + gate[None, :, None] * m[:, :, t]
        return y
    return run


@pytest.mark.parametrize("kind", ["no_current", "window_plus_one", "gate_on_local"])
def test_decode_layer_pins_catch_planted_mistakes(kind):
    q, k, v, lam, eta, g = rand_inputs(45, B=1, T=24, dk=4, dv=3)
    W, scale = 5, 0.7
    mut = _layer_mutant(kind)
    T = q.shape[2]
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref_l1 = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(band), scale=scale).numpy()
    gate = 1.0 / (1.0 + np.exp(-g))
    ref_l2 = gate[None, :, None, None] * brute_force_m(q, k, v, lam, eta, W)
    y1 = mut(q, k, v, lam, eta, g, W, scale)
    y0 = mut(q, k, v, lam, np.zeros_like(eta), g, W, scale)
    caught = np.max(np.abs(y0 - ref_l1)) > 1e-6 or np.max(np.abs((y1 - y0) - ref_l2)) > 1e-6
    assert caught
    # and the unmutated decoder passes the same two checks
    y1 = run_layer_decoder(q, k, v, lam, eta, g, W, scale)
    y0 = run_layer_decoder(q, k, v, lam, np.zeros_like(eta), g, W, scale)
    assert np.max(np.abs(y0 - ref_l1)) < 1e-12 and np.max(np.abs((y1 - y0) - ref_l2)) < 1e-12


# ---------------------------------------------------------------- backward of the scan

def _scan_loss(q, k, v, lam, eta, W, dm):
    return float(np.sum(O.tc_scan(q, k, v, lam, eta, W)[0] * dm))


@pytest.mark.parametrize("W,lam_kind", [(3, "u"), (1, "u"), (3, "0"), (3, "1"), (20, "u")])
def test_scan_backward_matches_central_differences(W, lam_kind):
    # every partial derivative against a central difference of the forward oracle
    q, k, v, lam, eta, _ = rand_inputs(50, B=1, H=2, T=12, dk=3, dv=3)
    lam = {"u": lam, "0": np.zeros(2), "1": np.ones(2)}[lam_kind]
    dm = np.random.default_rng(51).standard_normal(q.shape[:3] + (3,))
    gq, gk, gv, glam, geta = O.tc_scan_backward(q, k, v, lam, eta, W, dm)
    h = 1e-6
    for name, x, g in (("q", q, gq), ("k", k, gk), ("v", v, gv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _scan_loss(args["q"], args["k"], args["v"], lam, eta, W, dm)
            args[name] = xm
            lmn = _scan_loss(args["q"], args["k"], args["v"], lam, eta, W, dm)
            fd[i] = (lp - lmn) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)
    for hh in range(2):
        for name, g in (("lam", glam), ("eta", geta)):
            base = {"lam": lam, "eta": eta}[name]
            if name == "lam" and lam_kind == "0":
                continue  # lam = 0 sits on the edge of [0, 1]; checked one-sided below
            xp, xm = base.copy(), base.copy()
            xp[hh] += h
            xm[hh] -= h
            a = {"lam": lam, "eta": eta}
            a[name] = xp
            lp = _scan_loss(q, k, v, a["lam"], a["eta"], W, dm)
            a[name] = xm
            lmn = _scan_loss(q, k, v, a["lam"], a["eta"], W, dm)
            np.testing.assert_allclose(g[hh], (lp - lmn) / (2 * h), rtol=1e-6, atol=1e-8, err_msg=name)
    if lam_kind == "0":  # one-sided difference at lam = 0 (forward differences, second order)
        for hh in range(2):
            l1, l2 = lam.copy(), lam.copy()
            l1[hh], l2[hh] = h, 2 * h
            f0 = _scan_loss(q, k, v, lam, eta, W, dm)
            f1 = _scan_loss(q, k, v, l1, eta, W, dm)
            f2 = _scan_loss(q, k, v, l2, eta, W, dm)
            np.testing.assert_allclose(glam[hh], (-3 * f0 + 4 * f1 - f2) / (2 * h), rtol=1e-5, atol=1e-7)


def test_scan_backward_lambda_one_matches_autograd_of_cumulative_sum():
    # lam = 1: m_t = eta q_t sum_{i <= t-W} k_i v_i^T, a cumsum; torch autograd of that formula
    q, k, v, _, eta, _ = rand_inputs(52, B=2, H=2, T=30, dk=4, dv=5)
    W = 6
    dm = np.random.default_rng(53).standard_normal(q.shape[:3] + (5,))
    gq, gk, gv, _, geta = O.tc_scan_backward(q, k, v, np.ones(2), eta, W, dm)
    tq, tk, tv, te = (torch.tensor(a, requires_grad=True) for a in (q, k, v, eta))
    kv = torch.einsum("bhti,bhtj->bhtij", tk, tv)
    S = torch.cumsum(kv, dim=2)  # S[:, :, i] = sum_{j <= i} k_j v_j^T
    T = q.shape[2]
    Spad = torch.cat([torch.zeros_like(S[:, :, :W]), S[:, :, : T - W]], dim=2)  # state read at t
    m = te[None, :, None, None] * torch.einsum("bhti,bhtij->bhtj", tq, Spad)
    (m * torch.tensor(dm)).sum().backward()
    np.testing.assert_allclose(gq, tq.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gk, tk.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gv, tv.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(geta, te.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_scan_backward_scaling_identities():
    # scaling q (or k) by c scales m by c: sum <q, dq> = sum <k, dk> = <dm, m>;
    # m is linear in eta: eta * deta = <dm, m>
    q, k, v, lam, eta, _ = rand_inputs(54, B=2, H=2, T=40, dk=4, dv=4)
    W = 5
    dm = np.random.default_rng(55).standard_normal(q.shape)
    m, _ = O.tc_scan(q, k, v, lam, eta, W)
    gq, gk, gv, _, geta = O.tc_scan_backward(q, k, v, lam, eta, W, dm)
    per_head = np.einsum("bhtd,bhtd->h", dm, m)
    np.testing.assert_allclose(np.einsum("bhtd,bhtd->h", q, gq), per_head, rtol=1e-12)
    np.testing.assert_allclose(np.einsum("bhtd,bhtd->h", k, gk), per_head, rtol=1e-12)
    np.testing.assert_allclose(np.einsum("bhtd,bhtd->h", v, gv), per_head, rtol=1e-12)
    np.testing.assert_allclose(eta * geta, per_head, rtol=1e-12)


def _backward_mutant(kind):
    def run(q, k, v, lam, eta, W, dm):
        gq, gk, gv, glam, geta = O.tc_scan_backward(q, k, v, lam, eta, W, dm)
        if kind == "dk_one_token_late":
            gk = np.roll(gk, 1, axis=2)
        elif kind == "dlam_missing_a_term":
            glam = glam * 0.9
        elif kind == "dv_not_scaled_by_eta":
            gv = gv / eta[None, :, None, None]
        return gq, gk, gv, glam, geta
    return run


@pytest.mark.parametrize("kind", ["dk_one_token_late", "dlam_missing_a_term", "dv_not_scaled_by_eta"])
def test_scan_backward_pins_catch_planted_mistakes(kind):
    q, k, v, lam, eta, _ = rand_inputs(56, B=1, H=2, T=10, dk=2, dv=2)
    W = 2
    dm = np.random.default_rng(57).standard_normal(q.shape)
    gq, gk, gv, glam, geta = _backward_mutant(kind)(q, k, v, lam, eta, W, dm)
    h = 1e-6
    worst = 0.0
    for name, x, g in (("k", k, gk), ("v", v, gv)):
        for i in [(0, 0, 0, 0), (0, 1, 3, 1), (0, 0, 5, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            a = {"k": k, "v": v}
            a[name] = xp
            lp = _scan_loss(q, a["k"], a["v"], lam, eta, W, dm)
            a[name] = xm
            lmn = _scan_loss(q, a["k"], a["v"], lam, eta, W, dm)
            worst = max(worst, abs(g[i] - (lp - lmn) / (2 * h)))
    lp = _scan_loss(q, k, v, lam + np.array([h, 0]), eta, W, dm)
    lmn = _scan_loss(q, k, v, lam - np.array([h, 0]), eta, W, dm)
    worst = max(worst, abs(glam[0] - (lp - lmn) / (2 * h)))
    assert worst > 1e-4


def _gated_loss(q, k, v, lam, eta, g, W, dy):
    m = O.tc_scan(q, k, v, lam, eta, W)[0]
    return float(np.sum(O.sigmoid(g)[None, :, None, None] * m * dy))


def test_gated_read_backward_matches_central_differences():
    q, k, v, lam, eta, g = rand_inputs(60, B=2, H=2, T=11, dk=3, dv=2)
    g = np.array([0.7, -1.9])
    W = 3
    dy = np.random.default_rng(61).standard_normal(q.shape[:3] + (2,))
    gq, gk, gv, glam, geta, gg = O.tc_gated_read_backward(q, k, v, lam, eta, g, W, dy)
    h = 1e-6
    for name, x, gr in (("q", q, gq), ("k", k, gk), ("v", v, gv)):
        for i in [(0, 0, 5, 0), (1, 1, 9, 1), (0, 1, 2, 1), (1, 0, 0, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            a = {"q": q, "k": k, "v": v}
            a[name] = xp
            lp = _gated_loss(a["q"], a["k"], a["v"], lam, eta, g, W, dy)
            a[name] = xm
            lmn = _gated_loss(a["q"], a["k"], a["v"], lam, eta, g, W, dy)
            np.testing.assert_allclose(gr[i], (lp - lmn) / (2 * h), rtol=1e-6, atol=1e-9, err_msg=name)
    for hh in range(2):
        for name, gr in (("lam", glam), ("eta", geta), ("g", gg)):
            a = {"lam": lam.copy(), "eta": eta.copy(), "g": g.copy()}
            a[name][hh] += h
            lp = _gated_loss(q, k, v, a["lam"], a["eta"], a["g"], W, dy)
            a[name][hh] -= 2 * h
            lmn = _gated_loss(q, k, v, a["lam"], a["eta"], a["g"], W, dy)
            np.testing.assert_allclose(gr[hh], (lp - lmn) / (2 * h), rtol=1e-6, atol=1e-9, err_msg=name)


def test_gated_read_backward_gate_limits():
    # a wide-open gate passes the read's gradients through with dg -> 0; a
    # closed gate stops every gradient
    q, k, v, lam, eta, _ = rand_inputs(62, B=1, H=2, T=9, dk=2, dv=2)
    dy = np.random.default_rng(63).standard_normal(q.shape)
    ref = O.tc_scan_backward(q, k, v, lam, eta, 2, dy)
    out = O.tc_gated_read_backward(q, k, v, lam, eta, np.array([40.0, 40.0]), 2, dy)
    for a, b in zip(out[:5], ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    assert np.all(np.abs(out[5]) < 1e-15)
    out = O.tc_gated_read_backward(q, k, v, lam, eta, np.array([-800.0, -800.0]), 2, dy)
    assert all(np.all(a == 0) for a in out)


def test_gated_read_backward_pin_catches_sigmoid_for_its_derivative():
    q, k, v, lam, eta, _ = rand_inputs(64, B=1, H=1, T=8, dk=2, dv=2)
    g = np.array([0.3])
    dy = np.random.default_rng(65).standard_normal(q.shape)
    m = O.tc_scan(q, k, v, lam, eta, 2)[0]
    wrong = O.sigmoid(g) * np.einsum("bhtd,bhtd->h", dy, m)
    h = 1e-6
    fd = (_gated_loss(q, k, v, lam, eta, g + h, 2, dy) - _gated_loss(q, k, v, lam, eta, g - h, 2, dy)) / (2 * h)
    assert abs(wrong[0] - fd) > 1e-3

