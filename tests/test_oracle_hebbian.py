"""Pins of the Hebbian gated-MLP oracle.

Page: "Hebbian-memory MLP stores facts in a Transformer without training"
(mo.ai.kr): the gated feature map, the Hebbian output matrix, the storage
definition and the capacity trend.  CPU only.
"""
import numpy as np
import pytest

from oracle import hebbian as Hb


def unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def test_feature_kernel_mean_is_squared_inner_product():
    # E over Gaussian A, G of <phi(x), phi(y)> is m <x, y>^2 (A and G are
    # independent, E[(a.x)(a.y)] = <x, y>): a closed form the map must meet
    rng = np.random.default_rng(1)
    d, m = 8, 200000
    x, y = unit_rows(rng, 2, d)
    A, G = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    fx, fy = Hb.features(x[None], A, G)[0], Hb.features(y[None], A, G)[0]
    est = float(fx @ fy) / m
    want = float(x @ y) ** 2
    # the per-feature product has variance <= 9 for unit vectors: 4 sigma band
    assert abs(est - want) < 4 * 3 / np.sqrt(m)
    assert abs(float(fx @ fx) / m - 1.0) < 4 * 3 / np.sqrt(m)  # <x, x>^2 = 1


def test_write_is_the_sum_of_outer_products():
    rng = np.random.default_rng(2)
    F, d, m = 7, 5, 11
    K, V = unit_rows(rng, F, d), unit_rows(rng, F, d)
    f = rng.permutation(F)
    A, G = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    B = Hb.hebbian_write(K, V, f, A, G)
    want = np.zeros((d, m))
    for i in range(F):
        a, g = A @ K[i], G @ K[i]
        want += np.outer(V[f[i]], [a[c] * g[c] for c in range(m)])
    np.testing.assert_allclose(B, want / F, rtol=1e-13, atol=1e-15)


def test_read_is_the_kernel_weighted_sum_of_values():
    # MLP(q) = (1/F) sum_i <phi(k_i), phi(q)> v_f(i): the page's reading of the MLP
    rng = np.random.default_rng(3)
    F, d, m = 9, 6, 40
    K, V = unit_rows(rng, F, d), unit_rows(rng, F, d)
    f = rng.permutation(F)
    A, G = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    B = Hb.hebbian_write(K, V, f, A, G)
    q = unit_rows(rng, 1, d)
    out = Hb.hebbian_read(q, B, A, G)[0]
    fk, fq = Hb.features(K, A, G), Hb.features(q, A, G)[0]
    want = sum((fk[i] @ fq) * V[f[i]] for i in range(F)) / F
    np.testing.assert_allclose(out, want, rtol=1e-12)


def test_few_facts_are_all_stored_and_many_are_not():
    rng = np.random.default_rng(4)
    d, m = 32, 512
    A, G = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    K, V = unit_rows(rng, 8, d), unit_rows(rng, 8, d)
    assert Hb.stored_fraction(K, V, rng.permutation(8), A, G) == 1.0
    F = 20000  # far past m d / log F
    K, V = unit_rows(rng, F, d), unit_rows(rng, F, d)
    assert Hb.stored_fraction(K, V, rng.permutation(F), A, G) < 0.5


def test_capacity_falls_as_facts_pile_up():
    rng = np.random.default_rng(5)
    d, m = 16, 256
    A, G = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    fr = []
    for F in (64, 512, 4096):
        K, V = unit_rows(rng, F, d), unit_rows(rng, F, d)
        fr.append(Hb.stored_fraction(K, V, np.arange(F), A, G))
    assert fr[0] > fr[1] > fr[2]


def test_recall_argmax_ties_take_the_smallest_index():
    V = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    assert list(Hb.recall_argmax(np.array([[2.0, 1.0]]), V)) == [0]


def test_pin_catches_a_plain_product_feature_map():
    # phi(x) = (A x) * (A x) (G replaced by A) is a different kernel, with mean
    # m (1 + 2 <x, y>^2) for unit vectors: the kernel-mean pin rejects it
    rng = np.random.default_rng(6)
    d, m = 8, 200000
    x, y = unit_rows(rng, 2, d)
    A = rng.standard_normal((m, d))
    fx, fy = Hb.features(x[None], A, A)[0], Hb.features(y[None], A, A)[0]
    est = float(fx @ fy) / m
    assert abs(est - float(x @ y) ** 2) > 4 * 3 / np.sqrt(m)
