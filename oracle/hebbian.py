"""Float64 oracle of the Hebbian gated-MLP fact store.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Page: "Hebbian-memory MLP stores facts in a Transformer without training"
(mo.ai.kr), sections "Simple MLP construction" and "MLP storage capacity".

A fact set is keys k_1..k_F, values v_1..v_F and a map f: [F] -> [F] from key
index to value index.  With Gaussian A, G in R^{m x d} the gated feature map
is phi(x) = (A x) * (G x) (elementwise), the output matrix is
B = (1/F) sum_i v_{f(i)} phi(k_i)^T and the MLP is MLP(x) = B phi(x).  The
fact i is stored when, fed k_i, the output has its largest inner product with
v_{f(i)} among all value embeddings.

Readings taken where the page is silent: A and G have
independent N(0, 1) entries; a tie in the largest inner product counts as
the smallest index.
"""
from __future__ import annotations

import numpy as np

__all__ = ["features", "hebbian_write", "hebbian_read", "recall_argmax", "stored_fraction"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def features(x, A, G):
    """phi(x) = (A x) * (G x) for every row x of ``x`` [n, d]; returns [n, m]."""
    x, A, G = _f64(x), _f64(A), _f64(G)
    return (x @ A.T) * (x @ G.T)


def hebbian_write(K, V, f, A, G):
    """B = (1/F) sum_i v_{f(i)} phi(k_i)^T, [d_v, m]."""
    K, V = _f64(K), _f64(V)
    f = np.asarray(f)
    F = K.shape[0]
    return V[f].T @ features(K, A, G) / F


def hebbian_read(Q, B, A, G):
    """MLP(q) = B phi(q) for every row q of ``Q``; returns [n, d_v]."""
    return features(Q, A, G) @ _f64(B).T


def recall_argmax(out, V):
    """Index j of the largest <out_i, v_j> for every row (smallest j on a tie)."""
    scores = _f64(out) @ _f64(V).T
    return np.argmax(scores, axis=1)


def stored_fraction(K, V, f, A, G):
    """Fraction of the facts the MLP stores (the page's definition)."""
    B = hebbian_write(K, V, f, A, G)
    pred = recall_argmax(hebbian_read(K, B, A, G), V)
    return float(np.mean(pred == np.asarray(f)))
