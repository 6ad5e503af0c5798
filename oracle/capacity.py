"""Float64 oracle of the raw-memory capacity and recall diagnostic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page: "Tensor Cache: Eviction-conditioned Associative Memory for Transformers",
Methodology 1 (only pairs that leave the W-token window are written into A)
and the capacity diagnostic of the results (recall degrades as unrelated
associations pile up in the fixed-size matrix); the main contributions
contrast eviction conditioning with memories that ingest every token.

The diagnostic: a sequence of n_old "old" pairs followed by W "recent" pairs.
The eviction-conditioned memory is A after the sequence with window W (it
holds the old pairs only); the ingest-all memory is A after the same
sequence with every token written (window 1 and one trailing empty token).
Each old key reads its memory, r = k A, and the pair is recalled when the
read has its largest inner product with its own value among all the
sequence's values.

Readings: ingest-all is modelled by the same write with
window 1; a tie counts as the smallest index.
"""
from __future__ import annotations

import numpy as np

from . import tc

__all__ = ["tc_memory", "ingest_all_memory", "recall_hits"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def tc_memory(k, v, lam, eta, W):
    """A after the sequence with window W (the L2 matrix), [B, H, dk, dv]."""
    k, v = _f64(k), _f64(v)
    q = np.zeros_like(k)
    return tc.tc_scan(q, k, v, lam, eta, W)[1]


def ingest_all_memory(k, v, lam, eta):
    """A after writing every token of the sequence (window 1 and one trailing
    empty token, so the last pair is written too)."""
    k, v = _f64(k), _f64(v)
    zk = np.zeros(k.shape[:2] + (1, k.shape[3]))
    zv = np.zeros(v.shape[:2] + (1, v.shape[3]))
    return tc_memory(np.concatenate([k, zk], 2), np.concatenate([v, zv], 2), lam, eta, 1)


def recall_hits(A, k, v, n_old):
    """[B, H, n_old] booleans: the read k_j A of old pair j has its largest
    inner product with v_j among all the sequence's values."""
    A, k, v = _f64(A), _f64(k), _f64(v)
    R = np.einsum("bhni,bhiv->bhnv", k[:, :, :n_old], A)
    scores = np.einsum("bhnv,bhjv->bhnj", R, v)
    return np.argmax(scores, axis=-1) == np.arange(n_old)
