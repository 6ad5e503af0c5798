"""Parity of the capacity diagnostic (tc_scan_forward -> tc_memory_read ->
recall_argmax through the C ABI) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import diagnostics as Dg
from linear_attention_tensor_amd import inputs as I
from oracle import capacity as C
from tests._helpers import f32_dev, check, report

pytestmark = pytest.mark.gpu


def near_tie(A64, k64, v64, n_old):
    """[B, H, n_old]: the float64 top two scores are within rounding."""
    R = np.einsum("bhni,bhiv->bhnv", k64[:, :, :n_old], A64)
    s = np.sort(np.einsum("bhnv,bhjv->bhnj", R, v64), axis=-1)
    return (s[..., -1] - s[..., -2]) <= 1e-4 * (np.abs(s[..., -1]) + 1e-30)


@pytest.mark.parametrize("n_old,W,lam", [(16, 32, 1.0), (200, 64, 1.0), (500, 100, 0.99), (64, 1, 0.95)])
@pytest.mark.parametrize("ingest_all", [False, True])
def test_capacity_diagnostic_matches_oracle(n_old, W, lam, ingest_all):
    print(f"[case] capacity n_old={n_old} W={W} lam={lam} ingest_all={ingest_all}", flush=True)
    G, d = 6, 64
    x = I.draw_pairs(G, n_old + W, d, seed=n_old + W)
    k, v = f32_dev(x["k"]), f32_dev(x["v"])
    lam_t, eta_t = f32_dev(np.full(1, lam)), f32_dev(np.ones(1))
    A = Dg.memory_after(k, v, lam_t, eta_t, W, ingest_all=ingest_all)
    hits = Dg.recall_hits(A, k, v, n_old).cpu().numpy()
    k64, v64 = x["k"].astype(np.float64), x["v"].astype(np.float64)
    lam64 = np.full(1, np.float32(lam), np.float64)
    A_ref = C.ingest_all_memory(k64, v64, lam64, np.ones(1)) if ingest_all else C.tc_memory(k64, v64, lam64,
                                                                                             np.ones(1), W)
    check("A", A.cpu().numpy(), A_ref, 1e-5)
    want = C.recall_hits(A_ref, k64, v64, n_old)
    tie = near_tie(A_ref, k64, v64, n_old)
    assert np.array_equal(hits[~tie], want[~tie])
    print(f"[parity] recall {hits.mean():.4f} (oracle {want.mean():.4f}), {int(tie.sum())} near-ties", flush=True)
