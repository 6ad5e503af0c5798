"""Shared test helpers: seeded inputs -> torch tensors, error metrics."""
import numpy as np
import torch

# A row (the last axis) may miss the whole-tensor bar by at most this factor.
# Rounding spreads over every row about evenly, so a row far above the bar
# is a localized mistake (a wrong tile, slot or chunk), which the
# whole-tensor relative L2 alone would average away.
ROW_FACTOR = 3.0


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array from linear_attention_tensor_amd.inputs -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def f32_dev(arr, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_2 / ||ref||_2 in float64 over the whole tensor (0 if both are 0)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(x - ref)
    den = np.linalg.norm(ref)
    if den == 0:
        return float(num)
    return float(num / den)


def worst_row(x: np.ndarray, ref: np.ndarray):
    """Largest per-row error over the rows of the last axis, each relative to
    max(||ref row||, RMS row norm of ref); returns (value, flat row index).
    The floor keeps rows whose reference is nearly zero from dominating."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if x.size == 0:
        return 0.0, -1
    last = ref.shape[-1] if ref.ndim else 1
    d = (x - ref).reshape(-1, last)
    r = ref.reshape(-1, last)
    err = np.linalg.norm(d, axis=1)
    nrm = np.linalg.norm(r, axis=1)
    floor = float(np.sqrt(np.mean(nrm ** 2)))
    den = np.maximum(nrm, floor) if floor > 0 else np.ones_like(nrm)
    ratio = err / den
    i = int(np.argmax(ratio))
    return float(ratio[i]), i


def report(name, x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(x, ref)
    wr, wi = worst_row(x, ref)
    print(f"[parity] {name}: rel_l2={r:.3e} worst_row={wr:.3e}@{wi} "
          f"max_abs={np.max(np.abs(x - ref)) if x.size else 0:.3e}", flush=True)
    return r


def check(name, x, ref, tol, row_factor=ROW_FACTOR):
    """Assert the whole-tensor relative L2 <= tol and every row within
    row_factor * tol (see worst_row)."""
    r = report(name, x, ref)
    assert r <= tol, f"{name}: rel_l2 {r:.3e} > {tol:.1e}"
    wr, wi = worst_row(x, ref)
    assert wr <= row_factor * tol, f"{name}: row {wi} off by {wr:.3e} > {row_factor * tol:.1e}"
    return r


def same_bits(name, a: torch.Tensor, b: torch.Tensor):
    """Two results of the same call on the same inputs agree bit for bit."""
    a = a.detach().cpu()
    b = b.detach().cpu()
    assert a.shape == b.shape and a.dtype == b.dtype
    diff = int((a.view(torch.int32) != b.view(torch.int32)).sum()) if a.dtype == torch.float32 else \
        int((a != b).sum())
    print(f"[repeat] {name}: {diff} differing elements of {a.numel()}", flush=True)
    assert diff == 0, f"{name}: {diff} elements differ between two identical calls"
