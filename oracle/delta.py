"""Float64 oracle of the DeltaNet delta-rule memory.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page: "DeltaNet-family linear attention variants" (molayo1419.me).  The state
S is d_v x d_k (the core-identity section stores the summed outer products
|v><k| in a fixed d_v x d_k state), so a write is v k^T and a read is S q.

Readings taken where the page is silent: the output of
step t is read after that step's write, o_t = S_t q_t; S starts at zero unless
an initial state is passed.
"""
from __future__ import annotations

import numpy as np

__all__ = ["delta_scan", "additive_scan", "delta_scan_chunked", "reconstruction_loss", "delta_scan_backward"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def delta_scan(q, k, v, beta, S0=None):
    """Sequential delta rule: returns (o [B,H,T,dv], S_final [B,H,dv,dk]).

    "DeltaNet: writing the prediction error instead of the value": read the
    current prediction S_{t-1} k_t, then e_t = beta_t (v_t - S_{t-1} k_t) and
    S_t = S_{t-1} + e_t k_t^T, with beta_t in [0, 1].
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        pred = np.einsum("bhij,bhj->bhi", S, k[:, :, t, :])
        e = beta[:, :, t, None] * (v[:, :, t, :] - pred)
        S = S + e[..., :, None] * k[:, :, t, None, :]
        o[:, :, t, :] = np.einsum("bhij,bhj->bhi", S, q[:, :, t, :])
    return o, S


def additive_scan(q, k, v, S0=None):
    """Plain linear attention S_t = S_{t-1} + v_t k_t^T, o_t = S_t q_t.

    The additive-write section: a write adds v_t to what the key already
    returns instead of replacing it.  Used as the contrast case of the pins.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        S = S + v[:, :, t, :, None] * k[:, :, t, None, :]
        o[:, :, t, :] = np.einsum("bhij,bhj->bhi", S, q[:, :, t, :])
    return o, S


def reconstruction_loss(S, k, v):
    """1/2 ||S k - v||^2, the per-pair loss of the reconstruction-loss section."""
    r = _f64(S) @ _f64(k) - _f64(v)
    return 0.5 * float(r @ r)


def delta_scan_chunked(q, k, v, beta, C=64, S0=None):
    """Chunked evaluation of the delta rule, float64; equals ``delta_scan``.

    The page gives only the per-token rule; this form is derived from it.
    Inside a chunk entered with state S0, u_r = beta_r (v_r - S_{r-1} k_r) and
    S_{r-1} k_r = S0 k_r + sum_{i<r} <k_i, k_r> u_i.  With L the strictly lower
    triangle of K K^T this is (I + diag(beta) L) U = diag(beta) (V - K S0^T),
    so U = Tm (V - K S0^T) with Tm = (I + diag(beta) L)^-1 diag(beta).  Then
    O = Q S0^T + (Q K^T masked to i <= r) U and the exit state is S0 + U^T K.
    Kept apart from ``delta_scan`` only so a test can show the two agree.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t0 in range(0, T, C):
        L = min(C, T - t0)
        Q = q[:, :, t0 : t0 + L, :]
        K = k[:, :, t0 : t0 + L, :]
        V = v[:, :, t0 : t0 + L, :]
        bt = beta[:, :, t0 : t0 + L]
        KK = np.einsum("bhid,bhjd->bhij", K, K)
        strict = np.tril(np.ones((L, L)), -1)
        M = np.eye(L)[None, None] + bt[..., :, None] * KK * strict
        rhs = bt[..., :, None] * (V - np.einsum("bhrd,bhed->bhre", K, S))
        U = np.linalg.solve(M, rhs)
        QK = np.einsum("bhrd,bhid->bhri", Q, K) * np.tril(np.ones((L, L)))
        o[:, :, t0 : t0 + L, :] = np.einsum("bhrd,bhed->bhre", Q, S) + QK @ U
        S = S + np.einsum("bhre,bhrd->bhed", U, K)
    return o, S


def delta_scan_backward(q, k, v, beta, do, S0=None, dS_final=None):
    """Gradients of L = sum_t <do_t, o_t> + <dS_final, S_T> through ``delta_scan``.

    DeltaNet section of the page (beta is the learned write strength of every
    token).  Reverse mode through the per-token rule, with the states S_t of
    the forward pass kept: going backwards, dS (the adjoint of S_t) gathers
    do_t q_t^T and gives dq_t = S_t^T do_t; the write S_t = S_{t-1} + e_t k_t^T
    with e_t = beta_t (v_t - S_{t-1} k_t) sends de_t = dS k_t to
    dv_t = beta_t de_t and dbeta_t = <de_t, v_t - S_{t-1} k_t>, gives
    dk_t = dS^T e_t - beta_t S_{t-1}^T de_t, and leaves
    dS <- dS - beta_t de_t k_t^T for S_{t-1}.

    Returns (dq [B,H,T,dk], dk [B,H,T,dk], dv [B,H,T,dv], dbeta [B,H,T],
    dS0 [B,H,dv,dk]).
    """
    q, k, v, beta, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(do)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if S0 is None else _f64(S0).copy()
    states = [S.copy()]  # states[t] = S_{t-1}, the state before step t
    for t in range(T):
        e = beta[:, :, t, None] * (v[:, :, t] - np.einsum("bhij,bhj->bhi", S, k[:, :, t]))
        S = S + e[..., :, None] * k[:, :, t, None, :]
        states.append(S.copy())
    gq = np.zeros_like(q)
    gk = np.zeros_like(k)
    gv = np.zeros_like(v)
    gb = np.zeros_like(beta)
    dS = np.zeros((B, H, dv, dk)) if dS_final is None else _f64(dS_final).copy()
    for t in range(T - 1, -1, -1):
        S_t, S_prev = states[t + 1], states[t]
        dS = dS + do[:, :, t, :, None] * q[:, :, t, None, :]
        gq[:, :, t] = np.einsum("bhij,bhi->bhj", S_t, do[:, :, t])
        resid = v[:, :, t] - np.einsum("bhij,bhj->bhi", S_prev, k[:, :, t])
        e = beta[:, :, t, None] * resid
        de = np.einsum("bhij,bhj->bhi", dS, k[:, :, t])
        gv[:, :, t] = beta[:, :, t, None] * de
        gb[:, :, t] = np.einsum("bhi,bhi->bh", de, resid)
        gk[:, :, t] = (np.einsum("bhij,bhi->bhj", dS, e)
                       - beta[:, :, t, None] * np.einsum("bhij,bhi->bhj", S_prev, de))
        dS = dS - beta[:, :, t, None, None] * de[..., :, None] * k[:, :, t, None, :]
    return gq, gk, gv, gb, dS

