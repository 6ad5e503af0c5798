"""Shared test helpers: seeded inputs -> torch tensors, error metrics."""
import numpy as np
import torch


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


def report(name, x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(x, ref)
    print(f"[parity] {name}: rel_l2={r:.3e} max_abs={np.max(np.abs(x - ref)) if x.size else 0:.3e}", flush=True)
    return r
