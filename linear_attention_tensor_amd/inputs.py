"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU oracle.

This module holds no arithmetic of the method itself: it only draws random
numbers, normalises key rows (part of the input distribution, not of the
memory) and rounds to the storage dtype.  Both the HIP path and the oracle
receive what it produces, so a mismatch between them can only come from the
arithmetic on either side.

Recipe (the pages give no workload values; the shapes follow the five
workloads this library is measured on):

* ``numpy.random.Generator(PCG64(seed))``;
* draw order: q, k, v as float64 N(0, 1/d) (std 1/sqrt(d)); k rows
  L2-normalised in float64; then per head lambda, eta, g; then
  beta = logistic(N(0,1)) per (b, h, t);
* cast to float32, or to bfloat16 with round-to-nearest-even; the oracle gets
  the rounded values upcast to float64.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "draw_cotangent",
    "draw_facts",
    "draw_pairs",
    "FactWorkload",
    "FACT_WORKLOADS",
    "bf16_round_bits",
    "bf16_bits_to_f64",
    "round_to_dtype",
    "draw",
    "draw_decode_position",
    "decode_scalars",
    "draw_ring",
    "storage_to_f64",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    W: int
    dtype: str  # "f32" or "bf16" (input dtype; state and outputs are fp32)
    seed: int
    lam: tuple  # ("fixed", x) or ("uniform", lo, hi)
    eta: tuple
    chunk: int = 64
    steps: int = 0  # decode steps (streaming workload only)


# The five workloads: tiny single head (fp32), batched prefill scan (fp32),
# fused layer (bf16), streaming decode (bf16), delta-rule scan (bf16).
WORKLOADS = {
    "tiny_scan_f32": Workload("tiny_scan_f32", 1, 1, 256, 16, 32, "f32", 101,
                              ("fixed", 0.95), ("fixed", 0.5)),
    "prefill_scan_f32": Workload("prefill_scan_f32", 4, 8, 4096, 64, 512, "f32", 102,
                                 ("uniform", 0.9, 0.999), ("uniform", 0.1, 1.0)),
    "fused_layer_bf16": Workload("fused_layer_bf16", 1, 16, 32768, 128, 1024, "bf16", 103,
                                 ("uniform", 0.95, 0.999), ("uniform", 0.1, 1.0)),
    "decode_bf16": Workload("decode_bf16", 64, 32, 0, 128, 2048, "bf16", 104,
                            ("uniform", 0.95, 0.999), ("uniform", 0.1, 1.0), steps=4096),
    "delta_scan_bf16": Workload("delta_scan_bf16", 2, 16, 16384, 128, 0, "bf16", 105,
                                ("fixed", 1.0), ("fixed", 1.0)),
    # the delta scan's backward: same B, H, T; float32 inputs with d = 64
    "delta_backward_f32": Workload("delta_backward_f32", 2, 16, 16384, 64, 0, "f32", 106,
                                   ("fixed", 1.0), ("fixed", 1.0)),
}


def bf16_round_bits(x) -> np.ndarray:
    """Round float values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_dtype(x: np.ndarray, dtype: str):
    """Return (storage array, float64 view of the stored values).

    storage is float32 for "f32" and uint16 bfloat16 bits for "bf16".
    """
    if dtype == "f32":
        s = np.ascontiguousarray(x, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = bf16_round_bits(x)
        return s, bf16_bits_to_f64(s)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw_scalar(rng: np.random.Generator, spec: tuple, n: int) -> np.ndarray:
    if spec[0] == "fixed":
        return np.full(n, float(spec[1]), dtype=np.float64)
    if spec[0] == "uniform":
        return rng.uniform(spec[1], spec[2], size=n)
    raise ValueError(spec)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    n[n == 0] = 1.0
    return x / n


def draw(B: int, H: int, T: int, d: int, *, seed: int, dtype: str = "f32",
         lam=("uniform", 0.9, 0.999), eta=("uniform", 0.1, 1.0),
         dv: Optional[int] = None, normalize_keys: bool = True) -> dict:
    """Draw one batch of inputs in the fixed order of the recipe above.

    Returns a dict with storage arrays ``q, k, v`` (float32 or uint16 bf16
    bits), their float64 views ``q64, k64, v64``, float32 per-head ``lam,
    eta, g`` and float32 ``beta`` [B, H, T].  Scalars are float32 on both
    sides (the oracle upcasts the float32 values).
    """
    dv = d if dv is None else dv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    k = rng.standard_normal((B, H, T, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, T, dv)) / np.sqrt(dv)
    if normalize_keys:
        k = _unit_rows(k)
    lam_h = _draw_scalar(rng, lam, H).astype(np.float32)
    eta_h = _draw_scalar(rng, eta, H).astype(np.float32)
    g_h = rng.standard_normal(H).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))).astype(np.float32)
    out = {"dtype": dtype, "lam": lam_h, "eta": eta_h, "g": g_h, "beta": beta}
    for name, arr in (("q", q), ("k", k), ("v", v)):
        s, f = round_to_dtype(arr, dtype)
        out[name] = s
        out[name + "64"] = f
    return out


def draw_cotangent(B: int, H: int, T: int, dv: int, *, seed: int) -> np.ndarray:
    """Upstream gradient dm [B, H, T, dv] of the L2 read: float32 N(0, 1/dv),
    drawn from PCG64([seed, 1 << 42]) so it is independent of ``draw``."""
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 42]))
    return (rng.standard_normal((B, H, T, dv)) / np.sqrt(dv)).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class FactWorkload:
    """A fact-store workload: F facts, m gated features, dimension d."""
    name: str
    F: int
    m: int
    d: int
    seed: int


FACT_WORKLOADS = {
    "hebbian_f32": FactWorkload("hebbian_f32", 16384, 4096, 128, 107),
}


def draw_facts(F: int, d: int, m: int, *, seed: int, n_values: Optional[int] = None) -> dict:
    """A fact set and a gated feature map, float32: keys and values uniform on
    the unit sphere, f a random map of keys to values (a permutation when
    n_values == F), A and G with N(0, 1) entries [m, d]."""
    nv = F if n_values is None else n_values
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 43]))
    K = _unit_rows(rng.standard_normal((F, d)))
    V = _unit_rows(rng.standard_normal((nv, d)))
    f = rng.permutation(F) if nv == F else rng.integers(0, nv, size=F)
    A = rng.standard_normal((m, d))
    G = rng.standard_normal((m, d))
    return {"K": K.astype(np.float32), "V": V.astype(np.float32), "f": f.astype(np.int32),
            "A": A.astype(np.float32), "G": G.astype(np.float32)}


def draw_pairs(groups: int, T: int, d: int, *, seed: int) -> dict:
    """Key-value pairs uniform on the unit sphere, float32 [groups, 1, T, d]
    (one head per group), for the capacity diagnostic."""
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 44]))
    k = _unit_rows(rng.standard_normal((groups, 1, T, d)))
    v = _unit_rows(rng.standard_normal((groups, 1, T, d)))
    return {"k": k.astype(np.float32), "v": v.astype(np.float32)}


def draw_workload(name: str, *, T: Optional[int] = None, B: Optional[int] = None,
                  H: Optional[int] = None) -> dict:
    """Inputs of a named workload (optionally with a shorter T / fewer B, H)."""
    w = WORKLOADS[name]
    return draw(B if B is not None else w.B, H if H is not None else w.H,
                T if T is not None else w.T, w.d, seed=w.seed, dtype=w.dtype,
                lam=w.lam, eta=w.eta)


def draw_decode_position(B: int, H: int, d: int, pos: int, *, seed: int = 104,
                         dtype: str = "bf16") -> dict:
    """Inputs (q, k, v) of one streaming position, drawn from PCG64([seed, pos]).

    Drawing per position keeps the streaming workload reproducible without a
    single huge draw; keys are L2-normalised like everywhere else.
    """
    rng = np.random.Generator(np.random.PCG64([seed, pos]))
    q = rng.standard_normal((B, H, d)) / np.sqrt(d)
    k = _unit_rows(rng.standard_normal((B, H, d)) / np.sqrt(d))
    v = rng.standard_normal((B, H, d)) / np.sqrt(d)
    out = {"dtype": dtype}
    for name, arr in (("q", q), ("k", k), ("v", v)):
        s, f = round_to_dtype(arr, dtype)
        out[name] = s
        out[name + "64"] = f
    return out


def decode_scalars(H: int, *, seed: int = 104, lam=("uniform", 0.95, 0.999),
                   eta=("uniform", 0.1, 1.0)) -> dict:
    rng = np.random.Generator(np.random.PCG64([seed, 1 << 40]))
    return {"lam": _draw_scalar(rng, lam, H).astype(np.float32),
            "eta": _draw_scalar(rng, eta, H).astype(np.float32)}


def draw_ring(B: int, H: int, W: int, d: int, *, seed: int = 104, dtype: str = "bf16"):
    """A full W-slot ring of keys and values (one generator per sequence b).

    Slot i holds the token at position i, so with pos = W every slot is
    occupied and the next step evicts slot 0.  Returns the storage arrays
    (ring_k, ring_v) [B, H, W, d]; ``storage_to_f64`` gives their values.
    """
    ks, vs = [], []
    for b in range(B):
        rng = np.random.Generator(np.random.PCG64([seed, 1 << 41, b]))
        k = _unit_rows(rng.standard_normal((H, W, d)) / np.sqrt(d))
        v = rng.standard_normal((H, W, d)) / np.sqrt(d)
        ks.append(round_to_dtype(k, dtype)[0])
        vs.append(round_to_dtype(v, dtype)[0])
    return np.stack(ks), np.stack(vs)


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(arr) if dtype == "bf16" else np.asarray(arr, np.float64)
