"""Float64 oracle of the Tensor Cache two-level memory.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Page: "Tensor Cache: Eviction-conditioned Associative Memory for Transformers",
Methodology 1 (two-level architecture) and Methodology 2 (parallel scan).

Shapes: q, k [B, H, T, dk]; v [B, H, T, dv]; per-head lam, eta, g [H].
A is the per-head L2 matrix [B, H, dk, dv]; k (x) v is the outer product
k v^T and the read is the row vector q A.

Readings taken where the page is silent:

* the L1 window of query t holds the W most recent tokens, the current one
  included: positions max(0, t-W+1) .. t;
* at step t the token t-W leaves the window and is written into A
  (A <- lam A + eta k v^T), before the read m_t = q_t A of the same step; A
  decays only when a write happens, and starts at zero;
* the page's read r_t and the fused m_t are the same vector;
* the gate is the logistic function of one scalar per head, and the softmax
  scale is an explicit argument (1/sqrt(dk) by default).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "tc_scan",
    "tc_scan_rows",
    "TensorCacheDecoder",
    "window_softmax",
    "window_softmax_rows",
    "sigmoid",
    "tc_fused",
    "tc_fused_rows",
    "window_softmax_backward",
    "tc_fused_backward",
    "tc_scan_chunked",
    "chunk_mean_scan",
    "tc_scan_backward",
    "tc_gated_read_backward",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def tc_scan(q, k, v, lam, eta, W):
    """Sequential per-token L2 memory: returns (m [B,H,T,dv], A_final [B,H,dk,dv]).

    Tensor Cache, Methodology 1, write and read bullets: when the ring
    buffer overwrites an entry, the displaced pair is written as
    A <- lam A + eta (k (x) v); every query reads q_t A.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lam = _f64(lam)[None, :, None, None]
    eta = _f64(eta)[None, :, None, None]
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    A = np.zeros((B, H, dk, dv))
    m = np.zeros((B, H, T, dv))
    for t in range(T):
        e = t - W  # the token that leaves the W-token window at step t
        if e >= 0:
            A = lam * A + eta * (k[:, :, e, :, None] * v[:, :, e, None, :])
        m[:, :, t, :] = np.einsum("bhi,bhij->bhj", q[:, :, t, :], A)
    return m, A


def tc_scan_rows(q, k, v, lam, eta, W, rows):
    """m at selected positions from the closed-form weighted sum.

    Unrolling the write recurrence from A = 0 gives
    m_t = sum_{i <= t-W} eta lam^((t-W)-i) <q_t, k_i> v_i,
    the weighted sum the page's parallel scan evaluates.  Costs O(t d) per row,
    so it serves for spot checks at full sequence length.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lam = _f64(lam)
    eta = _f64(eta)
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, len(rows), dv))
    for n, t in enumerate(rows):
        e = t - W
        if e < 0:
            continue
        expo = (e - np.arange(e + 1, dtype=np.float64))  # (t-W) - i, i = 0..e
        wts = eta[:, None] * np.power(lam[:, None], expo[None, :])  # [H, e+1]
        s = np.einsum("bhid,bhd->bhi", k[:, :, : e + 1, :], q[:, :, t, :])
        out[:, :, n, :] = np.einsum("bhi,bhij->bhj", s * wts[None], v[:, :, : e + 1, :])
    return out


class TensorCacheDecoder:
    """Streaming form with a literal W-slot ring (one token per call).

    Tensor Cache, Methodology 1: the L1 cache is a fixed-size KV ring buffer of
    the W most recent tokens; when it overwrites an occupied entry, the pair
    that was there is written into A; the query then reads q A.

    The ring is kept as explicit slots with an occupancy flag, a deliberately
    different code shape from ``tc_scan`` so that an off-by-one in either
    shows up when the two are compared.
    """

    def __init__(self, B, H, dk, dv, W, lam, eta):
        self.W = int(W)
        self.lam = _f64(lam)
        self.eta = _f64(eta)
        self.ring_k = np.zeros((B, H, W, dk))
        self.ring_v = np.zeros((B, H, W, dv))
        self.occupied = np.zeros((B, W), dtype=bool)
        self.A = np.zeros((B, H, dk, dv))
        self.pos = np.zeros(B, dtype=np.int64)

    @classmethod
    def from_state(cls, ring_k, ring_v, A, pos, W, lam, eta):
        B, H, _, dk = ring_k.shape
        dv = ring_v.shape[-1]
        dec = cls(B, H, dk, dv, W, lam, eta)
        dec.ring_k[...] = ring_k
        dec.ring_v[...] = ring_v
        dec.A[...] = A
        dec.pos[...] = pos
        for b in range(B):
            dec.occupied[b, : min(int(pos[b]), W)] = True
        return dec

    def step(self, q, k, v):
        """q, k [B,H,dk], v [B,H,dv] -> m [B,H,dv]; advances each sequence by one."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, _ = q.shape
        m = np.zeros((B, H, v.shape[-1]))
        for b in range(B):
            slot = int(self.pos[b] % self.W)
            if self.occupied[b, slot]:
                ke = self.ring_k[b, :, slot, :].copy()
                ve = self.ring_v[b, :, slot, :].copy()
                for h in range(H):
                    self.A[b, h] = self.lam[h] * self.A[b, h] + self.eta[h] * np.outer(ke[h], ve[h])
            self.ring_k[b, :, slot, :] = k[b]
            self.ring_v[b, :, slot, :] = v[b]
            self.occupied[b, slot] = True
            for h in range(H):
                m[b, h] = q[b, h] @ self.A[b, h]
            self.pos[b] += 1
        return m

    def step_layer(self, q, k, v, g, scale=None):
        """Full decode step of the layer: q, k [B,H,dk], v [B,H,dv], g [H] -> y [B,H,dv].

        Tensor Cache, Methodology 1: the step above (eviction into A, the new
        pair into its slot, the read m = q A), then exact softmax attention of
        q over the pairs the ring holds after the write (the W most recent
        tokens, the current one included), and the gated sum
        y = y_local + sigmoid(g) m.  Advances each sequence by one.
        """
        q64 = _f64(q)
        B, H, dk = q64.shape
        scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
        m = self.step(q, k, v)
        gate = sigmoid(g)
        y = np.zeros_like(m)
        for b in range(B):
            held = np.flatnonzero(self.occupied[b])
            for h in range(H):
                s = (self.ring_k[b, h, held, :] @ q64[b, h]) * scale
                p = np.exp(s - s.max())
                p /= p.sum()
                y[b, h] = p @ self.ring_v[b, h, held, :] + gate[h] * m[b, h]
        return y


def window_softmax(q, k, v, W, scale):
    """L1 output: exact softmax attention over the W most recent tokens.

    Tensor Cache, Methodology 1, L1 bullet.  Query t attends to positions
    max(0, t-W+1) .. t with scores scale <q_t, k_j>; the max-subtracted
    softmax is only the usual overflow guard, it does not change the value.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, _ = q.shape
    y = np.zeros((B, H, T, v.shape[-1]))
    for t in range(T):
        lo = max(0, t - W + 1)
        s = np.einsum("bhjd,bhd->bhj", k[:, :, lo : t + 1, :], q[:, :, t, :]) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        y[:, :, t, :] = np.einsum("bhj,bhjd->bhd", p, v[:, :, lo : t + 1, :])
    return y


def window_softmax_rows(q, k, v, W, scale, rows):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, _ = q.shape
    y = np.zeros((B, H, len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        lo = max(0, t - W + 1)
        s = np.einsum("bhjd,bhd->bhj", k[:, :, lo : t + 1, :], q[:, :, t, :]) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        y[:, :, n, :] = np.einsum("bhj,bhjd->bhd", p, v[:, :, lo : t + 1, :])
    return y


def sigmoid(g):
    g = _f64(g)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def tc_fused(q, k, v, lam, eta, g, W, scale=None):
    """Fused layer y_t = y_local,t + sigmoid(g) m_t (Tensor Cache, Methodology 1, fusion).

    Returns (y [B,H,T,dv], A_final).
    """
    dk = np.shape(q)[-1]
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    y_loc = window_softmax(q, k, v, W, scale)
    m, A = tc_scan(q, k, v, lam, eta, W)
    return y_loc + sigmoid(g)[None, :, None, None] * m, A


def tc_fused_rows(q, k, v, lam, eta, g, W, rows, scale=None):
    dk = np.shape(q)[-1]
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    y_loc = window_softmax_rows(q, k, v, W, scale, rows)
    m = tc_scan_rows(q, k, v, lam, eta, W, rows)
    return y_loc + sigmoid(g)[None, :, None, None] * m


def _powers(lam, e):
    """lam ** e elementwise for integer e >= 0, with 0 ** 0 = 1."""
    return np.power(lam, e)


def tc_scan_chunked(q, k, v, lam, eta, W, C=64):
    """The chunked weighted-sum scan, float64; equals ``tc_scan`` up to rounding.

    Tensor Cache, Methodology 2: the parallel weighted-sum scan equals the
    sequential per-token writes.  With s = t - W the read is
    o_s = eta sum_{j <= s} lam^(s-j) <q_{s+W}, k_j> v_j, linear attention with
    a scalar decay whose query stream is shifted by W.  Per chunk n of C
    positions s = nC + r with entering state S_n (writes j < nC):

        o_r   = lam^(r+1) q'_r S_n + eta sum_{c <= r} lam^(r-c) <q'_r, k_c> v_c
        S_n+1 = lam^C S_n + eta sum_c lam^(C-1-c) k_c v_c^T

    This is the algebra the GPU kernels use; it is kept here, separately
    from ``tc_scan``, only so a test can show the two agree.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    lam = _f64(lam)
    eta = _f64(eta)
    m = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dk, dv))
    n_act = max(T - W, 0)
    r_idx = np.arange(C)
    for s0 in range(0, n_act, C):
        L = min(C, n_act - s0)
        r = r_idx[:L]
        Qp = q[:, :, s0 + W : s0 + W + L, :]
        Kc = k[:, :, s0 : s0 + L, :]
        Vc = v[:, :, s0 : s0 + L, :]
        gamma = _powers(lam[:, None], (r + 1)[None, :])  # [H, L]
        diff = r[:, None] - r[None, :]
        D = np.where(diff >= 0, _powers(lam[:, None, None], np.maximum(diff, 0)[None]), 0.0)
        inter = gamma[None, :, :, None] * np.einsum("bhrd,bhde->bhre", Qp, S)
        P = np.einsum("bhrd,bhcd->bhrc", Qp, Kc) * D[None] * eta[None, :, None, None]
        intra = np.einsum("bhrc,bhce->bhre", P, Vc)
        m[:, :, s0 + W : s0 + W + L, :] = inter + intra
        decay_c = _powers(lam[:, None], (L - 1 - r)[None, :]) * eta[:, None]  # [H, L]
        S = _powers(lam, L)[None, :, None, None] * S + np.einsum(
            "bhcd,bhc,bhce->bhde", Kc, np.broadcast_to(decay_c[None], (B, H, L)), Vc)
    return m, S


def chunk_mean_scan(q, k, v, lam, eta, W, C=64):
    """The naive chunk shortcut the page warns about (negative control only).

    Tensor Cache, Methodology 2: summarising a chunk by its means writes
    C * mean(k) (x) mean(v), which carries C^2 - C cross-token products
    k_i (x) v_j (i != j) that sequential writes never form.  Here each chunk of
    evicted tokens is written as one decayed write of that summary, and the
    reads of the chunk see the state after it.  Used only to show the pins
    reject it.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    lam = _f64(lam)[None, :, None, None]
    eta = _f64(eta)[None, :, None, None]
    m = np.zeros((B, H, T, dv))
    A = np.zeros((B, H, dk, dv))
    n_act = max(T - W, 0)
    for s0 in range(0, n_act, C):
        L = min(C, n_act - s0)
        kb = k[:, :, s0 : s0 + L, :].mean(axis=2)
        vb = v[:, :, s0 : s0 + L, :].mean(axis=2)
        A = np.power(lam, L) * A + eta * L * (kb[..., :, None] * vb[..., None, :])
        m[:, :, s0 + W : s0 + W + L, :] = np.einsum(
            "bhtd,bhde->bhte", q[:, :, s0 + W : s0 + W + L, :], A)
    return m, A


def tc_scan_backward(q, k, v, lam, eta, W, dm):
    """Gradients of L = sum <dm, m> through the L2 read m of ``tc_scan``.

    Tensor Cache, Methodology 1 (the write A <- lam A + eta k v^T on
    eviction, the read m_t = q_t A) and Methodology 2 (lam, eta are learned
    per head).  Reverse-mode through the sequential recurrence: the states
    A_t of the forward pass are kept, and dA accumulates q_t dm_t^T going
    backwards; a write at step t (token e = t - W) sends
    eta dA v_e to k_e, eta dA^T k_e to v_e, <dA, A_{t-1}> to lam and
    <dA, k_e v_e^T> to eta, and then dA <- lam dA.  A_final takes no
    upstream gradient.

    Returns (dq [B,H,T,dk], dk [B,H,T,dk], dv [B,H,T,dv], dlam [H], deta [H]);
    dlam and deta are summed over the batch.
    """
    q, k, v, dm = _f64(q), _f64(k), _f64(v), _f64(dm)
    lam, eta = _f64(lam), _f64(eta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    lm = lam[None, :, None, None]
    et = eta[None, :, None, None]
    A = np.zeros((B, H, dk, dv))
    states = []  # A_t after step t
    for t in range(T):
        if t >= W:
            e = t - W
            A = lm * A + et * np.einsum("bhi,bhj->bhij", k[:, :, e], v[:, :, e])
        states.append(A.copy())
    gq = np.zeros_like(q)
    gk = np.zeros_like(k)
    gv = np.zeros_like(v)
    glam = np.zeros((B, H))
    geta = np.zeros((B, H))
    dA = np.zeros((B, H, dk, dv))
    for t in range(T - 1, -1, -1):
        gq[:, :, t] = np.einsum("bhij,bhj->bhi", states[t], dm[:, :, t])
        dA = dA + np.einsum("bhi,bhj->bhij", q[:, :, t], dm[:, :, t])
        if t >= W:
            e = t - W
            prev = states[t - 1] if t >= 1 else np.zeros_like(dA)
            glam += np.einsum("bhij,bhij->bh", dA, prev)
            kv = np.einsum("bhi,bhj->bhij", k[:, :, e], v[:, :, e])
            geta += np.einsum("bhij,bhij->bh", dA, kv)
            gk[:, :, e] += et[..., 0] * np.einsum("bhij,bhj->bhi", dA, v[:, :, e])
            gv[:, :, e] += et[..., 0] * np.einsum("bhij,bhi->bhj", dA, k[:, :, e])
            dA = lm * dA
    return gq, gk, gv, glam.sum(axis=0), geta.sum(axis=0)


def tc_gated_read_backward(q, k, v, lam, eta, g, W, dy):
    """Gradients of L = sum <dy, sigmoid(g) m> through the L2 branch of the
    fused layer y = y_local + sigmoid(g) m (Tensor Cache, Methodology 1,
    fusion; g is learned per head).  y_local does not depend on lam, eta, g;
    its own gradients are not part of this function.

    Chain rule: the read's cotangent is dm = sigmoid(g) dy; the gate's is
    dg = sigmoid(g) (1 - sigmoid(g)) sum_{b,t} <dy_t, m_t>.

    Returns (dq, dk, dv, dlam, deta, dg); per-head terms summed over the batch.
    """
    dy = _f64(dy)
    s = sigmoid(g)
    gq, gk, gv, glam, geta = tc_scan_backward(q, k, v, lam, eta, W, s[None, :, None, None] * dy)
    m, _ = tc_scan(q, k, v, lam, eta, W)
    gg = s * (1.0 - s) * np.einsum("bhtd,bhtd->h", dy, m)
    return gq, gk, gv, glam, geta, gg


def window_softmax_backward(q, k, v, W, scale, dy):
    """Gradients of L = sum_t <dy_t, y_local,t> for the window softmax of
    window_softmax (Tensor Cache, Methodology 1, L1 cache; the pages give no
    backward, this is reverse mode through that definition).

    Per query t with window J = max(0, t-W+1) .. t, scores s_j = scale
    <q_t, k_j>, weights p = softmax(s) and y = sum_j p_j v_j:
      dv_j += p_j dy_t;
      dp_j = <dy_t, v_j>;  ds_j = p_j (dp_j - sum_i p_i dp_i);
      dq_t = scale sum_j ds_j k_j;  dk_j += scale ds_j q_t.
    Returns (dq, dk, dv).
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, T, _ = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t in range(T):
        lo = max(0, t - W + 1)
        kw, vw = k[:, :, lo : t + 1, :], v[:, :, lo : t + 1, :]
        s = np.einsum("bhjd,bhd->bhj", kw, q[:, :, t, :]) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        dv[:, :, lo : t + 1, :] += p[..., None] * dy[:, :, t, None, :]
        dp = np.einsum("bhjd,bhd->bhj", vw, dy[:, :, t, :])
        ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
        dq[:, :, t, :] = scale * np.einsum("bhj,bhjd->bhd", ds, kw)
        dk[:, :, lo : t + 1, :] += scale * ds[..., None] * q[:, :, t, None, :]
    return dq, dk, dv


def tc_fused_backward(q, k, v, lam, eta, g, W, dy, scale=None):
    """Gradients of L = sum_t <dy_t, y_t> for the fused layer y = y_local +
    sigmoid(g) m of tc_fused (Tensor Cache, Methodology 1, fusion): the two
    branches depend on q, k, v separately, so their gradients add; lam, eta
    and g enter only the L2 branch.

    Returns (dq, dk, dv, dlam, deta, dg); per-head terms summed over the batch.
    """
    dk_ = np.shape(q)[-1]
    scale = 1.0 / math.sqrt(dk_) if scale is None else float(scale)
    wq, wk, wv = window_softmax_backward(q, k, v, W, scale, dy)
    gq, gk, gv, glam, geta, gg = tc_gated_read_backward(q, k, v, lam, eta, g, W, dy)
    return wq + gq, wk + gk, wv + gv, glam, geta, gg
