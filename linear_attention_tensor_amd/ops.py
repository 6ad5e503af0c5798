"""Torch-facing binding of libtc.so with the names of the C entry points.

Argument marshalling only: shape/dtype/contiguity checks, output and
workspace allocation through torch, ``data_ptr()`` and the current HIP stream
handed to the C ABI.  Every step of the computation runs in the library's
kernels; there is no other path.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import TC_BF16, TC_F32, check, lib

__all__ = ["tc_scan_forward", "tc_scan_forward_noalloc", "tc_scan_backward", "tc_decode_step", "tc_decode_layer_step",
           "tc_fused_layer", "tc_window_attention", "tc_window_attention_backward", "tc_fused_layer_backward", "delta_scan_forward", "delta_scan_backward", "hebbian_write", "hebbian_read",
           "tc_memory_read", "recall_argmax", "scan_backward_workspace",
           "scan_workspace", "fused_workspace", "delta_workspace"]

CHUNK = 64


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TC_F32
    if t.dtype == torch.bfloat16:
        return TC_BF16
    raise TypeError(f"inputs must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensor(name: str, t: torch.Tensor, shape, dtype=None, device=None) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None:
        _need(t.device == device, f"{name} is on {t.device}, expected {device}")


def _check_unit_interval(name: str, t: torch.Tensor) -> None:
    # Reading the check's result back synchronises with the device, which a stream
    # under graph capture forbids: there the check is skipped (as with
    # check_values=False, which latency-bound callers pass anyway).
    if not t.numel() or torch.cuda.is_current_stream_capturing():
        return
    bad = (t < 0) | (t > 1) | torch.isnan(t)
    if bool(bad.any()):
        raise ValueError(f"{name} must lie in [0, 1]")


def _qkv(q, k, v):
    _need(q.dim() == 4, "q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for n, t, s in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv))):
        _check_tensor(n, t, s, q.dtype, q.device)
    return B, H, T, dk, dv, dt


def scan_workspace(B, H, T, dk, dv, W, dtype_code) -> int:
    n = lib().tc_scan_workspace_bytes(B, H, T, dk, dv, W, CHUNK, dtype_code)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("tc_scan_workspace_bytes", _lib.TC_ERR_INVALID_ARG, _lib.last_error())
    return n


def fused_workspace(B, H, T, dk, dv, W, dtype_code) -> int:
    n = lib().tc_fused_workspace_bytes(B, H, T, dk, dv, W, CHUNK, dtype_code)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("tc_fused_workspace_bytes", _lib.TC_ERR_UNSUPPORTED, _lib.last_error())
    return n


def delta_workspace(B, H, T, dk, dv, dtype_code) -> int:
    n = lib().delta_scan_workspace_bytes(B, H, T, dk, dv, CHUNK, dtype_code)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("delta_scan_workspace_bytes", _lib.TC_ERR_INVALID_ARG, _lib.last_error())
    return n


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None


def tc_scan_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor,
                    eta: torch.Tensor, W: int, *, return_state: bool = True,
                    check_values: bool = True, m: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """L2 memory read m [B,H,T,dv] (fp32) and the final state A [B,H,dk,dv]."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("lam", lam, (H,), torch.float32, q.device)
    _check_tensor("eta", eta, (H,), torch.float32, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
    if m is None:
        m = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("m", m, (B, H, T, dv), torch.float32, q.device)
    A = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if return_state else None
    need = scan_workspace(B, H, T, dk, dv, W, dt)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().tc_scan_forward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lam), _ptr(eta), B, H, T, dk, dv,
                               W, CHUNK, _ptr(m), _ptr(A), _ptr(ws), ws.numel() if ws is not None else 0,
                               _stream())
    check("tc_scan_forward", st)
    return m, A


def tc_scan_forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor,
                            eta: torch.Tensor, W: int, *, m: torch.Tensor,
                            A_final: Optional[torch.Tensor] = None,
                            check_values: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """tc_scan_forward into caller-given outputs with the library's own scratch:
    nothing is allocated (m [B,H,T,dv] and A_final [B,H,dk,dv] or None)."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("lam", lam, (H,), torch.float32, q.device)
    _check_tensor("eta", eta, (H,), torch.float32, q.device)
    _check_tensor("m", m, (B, H, T, dv), torch.float32, q.device)
    if A_final is not None:
        _check_tensor("A_final", A_final, (B, H, dk, dv), torch.float32, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
    st = lib().tc_scan_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lam), _ptr(eta), B, H, T, dk,
                                       dv, W, CHUNK, _ptr(m), _ptr(A_final), _stream())
    check("tc_scan_forward_noalloc", st)
    return m, A_final


def scan_backward_workspace(B, H, T, dk, dv, W, dtype_code) -> int:
    n = lib().tc_scan_backward_workspace_bytes(B, H, T, dk, dv, W, CHUNK, dtype_code)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("tc_scan_backward_workspace_bytes", _lib.TC_ERR_UNSUPPORTED, _lib.last_error())
    return n


def tc_scan_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor,
                     eta: torch.Tensor, W: int, dm: torch.Tensor, *, g: Optional[torch.Tensor] = None,
                     check_values: bool = True, ws: Optional[torch.Tensor] = None):
    """Gradients of sum <dm, m> through the L2 read m: (dq, dk, dv, dlam, deta).

    With a per-head gate ``g`` [H], ``dm`` is the cotangent of sigmoid(g) m
    (the gated branch of the fused layer) and dg [H] is returned last.
    """
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("lam", lam, (H,), torch.float32, q.device)
    _check_tensor("eta", eta, (H,), torch.float32, q.device)
    _check_tensor("dm", dm, (B, H, T, dv), torch.float32, q.device)
    if g is not None:
        _check_tensor("g", g, (H,), torch.float32, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
    gq = torch.empty((B, H, T, dk), dtype=torch.float32, device=q.device)
    gk = torch.empty((B, H, T, dk), dtype=torch.float32, device=q.device)
    gv = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    glam = torch.empty((H,), dtype=torch.float32, device=q.device)
    geta = torch.empty((H,), dtype=torch.float32, device=q.device)
    gg = torch.empty((H,), dtype=torch.float32, device=q.device) if g is not None else None
    need = scan_backward_workspace(B, H, T, dk, dv, W, dt)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().tc_scan_backward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lam), _ptr(eta), _ptr(g), B, H, T, dk,
                                dv, W, CHUNK, _ptr(dm), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(glam), _ptr(geta),
                                _ptr(gg), _ptr(ws), ws.numel() if ws is not None else 0, _stream())
    check("tc_scan_backward", st)
    if g is not None:
        return gq, gk, gv, glam, geta, gg
    return gq, gk, gv, glam, geta


def tc_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ring_k: torch.Tensor,
                   ring_v: torch.Tensor, A: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor,
                   pos: torch.Tensor, W: int, *, m: Optional[torch.Tensor] = None,
                   check_values: bool = True) -> torch.Tensor:
    """One streaming step; updates ring_k, ring_v and A in place, returns m [B,H,dv].

    The caller advances ``pos`` (tokens already seen per sequence) afterwards.
    """
    _need(q.dim() == 3, "q must be [B, H, dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for n, t, s in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                    ("ring_k", ring_k, (B, H, W, dk)), ("ring_v", ring_v, (B, H, W, dv))):
        _check_tensor(n, t, s, q.dtype, q.device)
    _check_tensor("A", A, (B, H, dk, dv), torch.float32, q.device)
    _check_tensor("lam", lam, (H,), torch.float32, q.device)
    _check_tensor("eta", eta, (H,), torch.float32, q.device)
    _check_tensor("pos", pos, (B,), torch.int64, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
        if pos.numel() and not torch.cuda.is_current_stream_capturing() and bool((pos < 0).any()):
            raise ValueError("pos must be >= 0")
    if m is None:
        m = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("m", m, (B, H, dv), torch.float32, q.device)
    st = lib().tc_decode_step(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(ring_k), _ptr(ring_v), _ptr(A),
                              _ptr(lam), _ptr(eta), _ptr(pos), B, H, dk, dv, W, _ptr(m), _stream())
    check("tc_decode_step", st)
    return m


def tc_decode_layer_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ring_k: torch.Tensor,
                         ring_v: torch.Tensor, A: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor,
                         g: torch.Tensor, pos: torch.Tensor, W: int, *,
                         softmax_scale: Optional[float] = None, y: Optional[torch.Tensor] = None,
                         check_values: bool = True) -> torch.Tensor:
    """One full decode step of the layer; updates ring_k, ring_v and A in place and
    returns y [B,H,dv] = ring softmax attention + sigmoid(g) * L2 read.

    The caller advances ``pos`` (tokens already seen per sequence) afterwards.
    """
    _need(q.dim() == 3, "q must be [B, H, dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for n, t, s in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                    ("ring_k", ring_k, (B, H, W, dk)), ("ring_v", ring_v, (B, H, W, dv))):
        _check_tensor(n, t, s, q.dtype, q.device)
    _check_tensor("A", A, (B, H, dk, dv), torch.float32, q.device)
    for n, t in (("lam", lam), ("eta", eta), ("g", g)):
        _check_tensor(n, t, (H,), torch.float32, q.device)
    _check_tensor("pos", pos, (B,), torch.int64, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
        if pos.numel() and not torch.cuda.is_current_stream_capturing() and bool((pos < 0).any()):
            raise ValueError("pos must be >= 0")
    scale = 1.0 / math.sqrt(dk) if softmax_scale is None else float(softmax_scale)
    if y is None:
        y = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("y", y, (B, H, dv), torch.float32, q.device)
    st = lib().tc_decode_layer_step(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(ring_k), _ptr(ring_v), _ptr(A),
                                    _ptr(lam), _ptr(eta), _ptr(g), _ptr(pos), B, H, dk, dv, W, scale,
                                    _ptr(y), _stream())
    check("tc_decode_layer_step", st)
    return y


def tc_fused_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor,
                   eta: torch.Tensor, g: torch.Tensor, W: int, *, softmax_scale: Optional[float] = None,
                   return_state: bool = False, check_values: bool = True,
                   y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """y = sliding-window softmax attention + sigmoid(g) * L2 read; optionally A_final."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    for n, t in (("lam", lam), ("eta", eta), ("g", g)):
        _check_tensor(n, t, (H,), torch.float32, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
    scale = 1.0 / math.sqrt(dk) if softmax_scale is None else float(softmax_scale)
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("y", y, (B, H, T, dv), torch.float32, q.device)
    A = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if return_state else None
    need = fused_workspace(B, H, T, dk, dv, W, dt)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().tc_fused_layer(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lam), _ptr(eta), _ptr(g), B, H, T,
                              dk, dv, W, CHUNK, scale, _ptr(y), _ptr(A), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream())
    check("tc_fused_layer", st)
    return (y, A) if return_state else y


def tc_window_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: int, *,
                        softmax_scale: Optional[float] = None,
                        y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The L1 cache alone: exact softmax attention over the W most recent tokens, y [B,H,T,dv] fp32."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    scale = 1.0 / math.sqrt(dk) if softmax_scale is None else float(softmax_scale)
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("y", y, (B, H, T, dv), torch.float32, q.device)
    st = lib().tc_window_attention(_ptr(q), _ptr(k), _ptr(v), dt, B, H, T, dk, dv, W, scale, _ptr(y), _stream())
    check("tc_window_attention", st)
    return y


def tc_window_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: int, dy: torch.Tensor, *,
                                 softmax_scale: Optional[float] = None):
    """Gradients (dq, dk, dv) of sum <dy, y> for y = tc_window_attention(q, k, v, W)."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("dy", dy, (B, H, T, dv), torch.float32, q.device)
    scale = 1.0 / math.sqrt(dk) if softmax_scale is None else float(softmax_scale)
    n = lib().tc_window_attention_backward_workspace_bytes(B, H, T, dk, dv, W, dt)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("tc_window_attention_backward_workspace_bytes", _lib.TC_ERR_INVALID_ARG, _lib.last_error())
    ws = _ws(n, q.device)
    grads = [torch.empty((B, H, T, x), dtype=torch.float32, device=q.device) for x in (dk, dk, dv)]
    st = lib().tc_window_attention_backward(_ptr(q), _ptr(k), _ptr(v), dt, B, H, T, dk, dv, W, scale, _ptr(dy),
                                            *(_ptr(t) for t in grads), _ptr(ws), ws.numel() if ws is not None else 0,
                                            _stream())
    check("tc_window_attention_backward", st)
    return tuple(grads)


def tc_fused_layer_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: torch.Tensor, eta: torch.Tensor,
                            g: torch.Tensor, W: int, dy: torch.Tensor, *, softmax_scale: Optional[float] = None,
                            check_values: bool = True):
    """Gradients (dq, dk, dv, dlam, deta, dg) of sum <dy, y> for y = tc_fused_layer(...)."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    for n_, t in (("lam", lam), ("eta", eta), ("g", g)):
        _check_tensor(n_, t, (H,), torch.float32, q.device)
    _check_tensor("dy", dy, (B, H, T, dv), torch.float32, q.device)
    if check_values:
        _check_unit_interval("lam", lam)
    scale = 1.0 / math.sqrt(dk) if softmax_scale is None else float(softmax_scale)
    n = lib().tc_fused_layer_backward_workspace_bytes(B, H, T, dk, dv, W, CHUNK, dt)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("tc_fused_layer_backward_workspace_bytes", _lib.TC_ERR_UNSUPPORTED, _lib.last_error())
    ws = _ws(n, q.device)
    grads = [torch.empty((B, H, T, x), dtype=torch.float32, device=q.device) for x in (dk, dk, dv)]
    hg = [torch.empty((H,), dtype=torch.float32, device=q.device) for _ in range(3)]
    st = lib().tc_fused_layer_backward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lam), _ptr(eta), _ptr(g), B, H, T, dk,
                                       dv, W, CHUNK, scale, _ptr(dy), *(_ptr(t) for t in grads),
                                       *(_ptr(t) for t in hg), _ptr(ws), ws.numel() if ws is not None else 0,
                                       _stream())
    check("tc_fused_layer_backward", st)
    return tuple(grads) + tuple(hg)


def delta_scan_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor, *,
                       S0: Optional[torch.Tensor] = None, return_state: bool = False,
                       check_values: bool = True, o: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None):
    """Delta-rule outputs o [B,H,T,dv] (fp32); optionally S_final [B,H,dv,dk]."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("beta", beta, (B, H, T), torch.float32, q.device)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dv, dk), torch.float32, q.device)
    if check_values:
        _check_unit_interval("beta", beta)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("o", o, (B, H, T, dv), torch.float32, q.device)
    S = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device) if return_state else None
    need = delta_workspace(B, H, T, dk, dv, dt)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().delta_scan_forward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(beta), B, H, T, dk, dv, CHUNK,
                                  _ptr(S0), _ptr(o), _ptr(S), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream())
    check("delta_scan_forward", st)
    return (o, S) if return_state else o


def delta_scan_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                        do: torch.Tensor, *, S0: Optional[torch.Tensor] = None,
                        dS_final: Optional[torch.Tensor] = None, return_dS0: bool = False,
                        check_values: bool = True, ws: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dbeta[, dS0]) of sum <do, o> (+ <dS_final, S_final>)
    through delta_scan_forward; float32 or bfloat16 inputs, d in {16, 32, 64, 128}."""
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _check_tensor("beta", beta, (B, H, T), torch.float32, q.device)
    _check_tensor("do", do, (B, H, T, dv), torch.float32, q.device)
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None:
            _check_tensor(name, t, (B, H, dv, dk), torch.float32, q.device)
    if check_values:
        _check_unit_interval("beta", beta)
    gq = torch.empty((B, H, T, dk), dtype=torch.float32, device=q.device)
    gk = torch.empty((B, H, T, dk), dtype=torch.float32, device=q.device)
    gv = torch.empty((B, H, T, dv), dtype=torch.float32, device=q.device)
    gb = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    gS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device) if return_dS0 else None
    n = lib().delta_scan_backward_workspace_bytes(B, H, T, dk, dv, CHUNK, dt)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("delta_scan_backward_workspace_bytes", _lib.TC_ERR_UNSUPPORTED, _lib.last_error())
    if ws is None:
        ws = _ws(n, q.device)
    st = lib().delta_scan_backward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(beta), B, H, T, dk, dv, CHUNK, _ptr(S0),
                                   _ptr(do), _ptr(dS_final), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gb), _ptr(gS0),
                                   _ptr(ws), ws.numel() if ws is not None else 0, _stream())
    check("delta_scan_backward", st)
    return (gq, gk, gv, gb, gS0) if return_dS0 else (gq, gk, gv, gb)


def _f32_2d(name, t, shape0, d, device):
    _check_tensor(name, t, (shape0, d), torch.float32, device)


def hebbian_write(K: torch.Tensor, V: torch.Tensor, f: torch.Tensor, A: torch.Tensor, G: torch.Tensor, *,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """B^T [m, d] of the Hebbian gated-MLP store (B = (1/F) sum_i V[f[i]] phi(K[i])^T)."""
    F, d = K.shape
    m = A.shape[0]
    _f32_2d("K", K, F, d, K.device)
    _f32_2d("V", V, V.shape[0], d, K.device)
    _f32_2d("A", A, m, d, K.device)
    _f32_2d("G", G, m, d, K.device)
    _check_tensor("f", f, (F,), torch.int32, K.device)
    n = lib().hebbian_workspace_bytes(F, m, d)
    if n == _lib.SIZE_MAX:
        raise _lib.TCError("hebbian_workspace_bytes", _lib.TC_ERR_UNSUPPORTED, _lib.last_error())
    if ws is None:
        ws = _ws(n, K.device)
    Bt = torch.empty((m, d), dtype=torch.float32, device=K.device)
    st = lib().hebbian_write(_ptr(K), _ptr(V), _ptr(f), F, V.shape[0], _ptr(A), _ptr(G), m, d, _ptr(Bt), _ptr(ws),
                             ws.numel(), _stream())
    check("hebbian_write", st)
    return Bt


def hebbian_read(Q: torch.Tensor, A: torch.Tensor, G: torch.Tensor, Bt: torch.Tensor) -> torch.Tensor:
    """B phi(q) for every row q of Q [n, d]."""
    n, d = Q.shape
    m = A.shape[0]
    _f32_2d("Q", Q, n, d, Q.device)
    _f32_2d("A", A, m, d, Q.device)
    _f32_2d("G", G, m, d, Q.device)
    _f32_2d("Bt", Bt, m, d, Q.device)
    out = torch.empty((n, d), dtype=torch.float32, device=Q.device)
    check("hebbian_read", lib().hebbian_read(_ptr(Q), n, _ptr(A), _ptr(G), _ptr(Bt), m, d, _ptr(out), _stream()))
    return out


def tc_memory_read(Q: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """Q[g] A[g] for every group g: Q [groups, n, d], A [groups, d, d]."""
    groups, n, d = Q.shape
    _check_tensor("Q", Q, (groups, n, d), torch.float32, Q.device)
    _check_tensor("A", A, (groups, d, d), torch.float32, Q.device)
    out = torch.empty((groups, n, d), dtype=torch.float32, device=Q.device)
    check("tc_memory_read", lib().tc_memory_read(_ptr(Q), _ptr(A), groups, n, d, _ptr(out), _stream()))
    return out


def recall_argmax(R: torch.Tensor, V: torch.Tensor):
    """(arg, best): the candidate of V[g] [nc, d] with the largest inner product
    with each row of R[g] [nq, d] (smallest index on a tie), and that product."""
    groups, nq, d = R.shape
    nc = V.shape[1]
    _check_tensor("R", R, (groups, nq, d), torch.float32, R.device)
    _check_tensor("V", V, (groups, nc, d), torch.float32, R.device)
    arg = torch.empty((groups, nq), dtype=torch.int32, device=R.device)
    best = torch.empty((groups, nq), dtype=torch.float32, device=R.device)
    check("recall_argmax", lib().recall_argmax(_ptr(R), _ptr(V), groups, nq, nc, d, _ptr(arg), _ptr(best),
                                               _stream()))
    return arg, best

