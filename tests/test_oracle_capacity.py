"""Pins of the raw-memory capacity diagnostic oracle.

Page: "Tensor Cache", Methodology 1 (eviction-conditioned writes) and the
capacity diagnostic of the results.  CPU only.
"""
import numpy as np

from oracle import capacity as C


def unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_tc_memory_holds_exactly_the_evicted_pairs():
    rng = np.random.default_rng(1)
    n_old, W, d = 9, 5, 4
    k, v = unit(rng, (1, 2, n_old + W, d)), unit(rng, (1, 2, n_old + W, d))
    lam, eta = np.array([0.9, 1.0]), np.array([0.5, 2.0])
    A = C.tc_memory(k, v, lam, eta, W)
    for h in range(2):
        want = sum(eta[h] * lam[h] ** (n_old - 1 - i) * np.outer(k[0, h, i], v[0, h, i]) for i in range(n_old))
        np.testing.assert_allclose(A[0, h], want, rtol=1e-13, atol=1e-15)
    Aall = C.ingest_all_memory(k, v, lam, eta)
    T = n_old + W
    for h in range(2):
        want = sum(eta[h] * lam[h] ** (T - 1 - i) * np.outer(k[0, h, i], v[0, h, i]) for i in range(T))
        np.testing.assert_allclose(Aall[0, h], want, rtol=1e-13, atol=1e-15)


def test_orthonormal_keys_are_all_recalled():
    # d orthonormal keys, lam = 1: k_j A = eta v_j exactly
    d = 16
    rng = np.random.default_rng(2)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[None, None]  # rows orthonormal
    v = unit(rng, (1, 1, d, d))
    A = C.tc_memory(k, v, np.ones(1), np.ones(1), 1)
    # W = 1 leaves the last pair in the window; the others are recalled exactly
    assert C.recall_hits(A, k, v, d - 1).all()


def test_eviction_conditioning_protects_old_pairs_from_recent_interference():
    # recent pairs reuse the old keys with other values: the ingest-all memory
    # writes them too, and with decay they outweigh the old values, which it
    # loses; the eviction-conditioned memory holds the old pairs only
    rng = np.random.default_rng(3)
    d, n = 64, 8
    k_old = unit(rng, (1, 1, n, d))
    k = np.concatenate([k_old, k_old], axis=2)
    v = unit(rng, (1, 1, 2 * n, d))
    lam, eta = np.full(1, 0.9), np.ones(1)
    assert C.recall_hits(C.tc_memory(k, v, lam, eta, n), k, v, n).all()
    assert not C.recall_hits(C.ingest_all_memory(k, v, lam, eta), k, v, n).any()
    # without decay the two values of a key tie in weight: about half survive
    frac = C.recall_hits(C.ingest_all_memory(k, v, np.ones(1), eta), k, v, n).mean()
    assert 0.0 < frac < 1.0


def test_recall_falls_as_pairs_pile_up():
    rng = np.random.default_rng(4)
    d, W = 32, 16
    rates = []
    for n in (8, 64, 512):
        k, v = unit(rng, (8, 1, n + W, d)), unit(rng, (8, 1, n + W, d))
        A = C.tc_memory(k, v, np.ones(1), np.ones(1), W)
        rates.append(C.recall_hits(A, k, v, n).mean())
    assert rates[0] == 1.0 and rates[0] > rates[1] > rates[2]
