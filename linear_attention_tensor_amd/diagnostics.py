"""Raw-memory capacity and recall diagnostic on the GPU.

"Tensor Cache", Methodology 1 (only pairs that leave the W-token window are
written) and the capacity diagnostic of its results.  A sequence holds
n_old "old" pairs followed by W "recent" pairs; the eviction-conditioned
memory is A after the sequence with window W, the ingest-all memory writes
every token (window 1 and one trailing empty token).  Each old key reads its
memory (r = k A) and the pair is recalled when r has its largest inner
product with its own value among all the sequence's values.

Every step runs in libtc: the writes in tc_scan_forward, the reads in
tc_memory_read, the scores and their argmax in recall_argmax.  This module
only arranges the calls.
"""
from __future__ import annotations

import torch

from . import ops

__all__ = ["memory_after", "recall_hits", "capacity_point"]


def memory_after(k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor, W: int, *,
                 ingest_all: bool = False) -> torch.Tensor:
    """A [B, H, d, d] after the sequence k, v [B, H, T, d] (fp32): window W, or
    every token written when ``ingest_all``."""
    if ingest_all:
        pad = torch.zeros_like(k[:, :, :1])
        k = torch.cat([k, pad], dim=2)
        v = torch.cat([v, torch.zeros_like(v[:, :, :1])], dim=2)
        W = 1
    q = torch.zeros_like(k)
    _, A = ops.tc_scan_forward(q, k, v, lam, eta, W, return_state=True)
    return A


def recall_hits(A: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_old: int) -> torch.Tensor:
    """[B, H, n_old] booleans: old pair j is recalled from A."""
    B, H, T, d = k.shape
    R = ops.tc_memory_read(k[:, :, :n_old].reshape(B * H, n_old, d).contiguous(), A.reshape(B * H, d, d))
    arg, _ = ops.recall_argmax(R, v.reshape(B * H, T, d))
    idx = torch.arange(n_old, device=k.device, dtype=arg.dtype)
    return (arg == idx).reshape(B, H, n_old)


def capacity_point(k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor, W: int, n_old: int):
    """(eviction-conditioned, ingest-all) recall rates of the n_old old pairs."""
    tc = recall_hits(memory_after(k, v, lam, eta, W), k, v, n_old)
    ia = recall_hits(memory_after(k, v, lam, eta, W, ingest_all=True), k, v, n_old)
    return float(tc.float().mean()), float(ia.float().mean())
