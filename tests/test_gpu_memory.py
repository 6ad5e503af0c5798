"""Parity of the fact-memory entry points (hebbian_write, hebbian_read,
tc_memory_read, recall_argmax; C ABI, HIP kernels) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import hebbian as Hb
from tests._helpers import f32_dev, check, report

pytestmark = pytest.mark.gpu

TOL = 1e-5


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def f64(x):
    return np.asarray(x, np.float64)


def check_argmax(arg, R64, V64, label):
    """Exact where the float64 top two are apart by more than rounding can
    move them; elsewhere the pick must be one of the (near-)tied best."""
    scores = R64 @ V64.T
    top = np.sort(scores, axis=1)[:, -2:] if scores.shape[1] > 1 else np.concatenate([scores, scores], 1)
    scale = np.abs(top[:, 1]) + 1e-30
    clear = (top[:, 1] - top[:, 0]) > 1e-4 * scale
    want = np.argmax(scores, axis=1)
    assert np.array_equal(arg[clear], want[clear]), f"{label}: argmax differs on clear cases"
    picked = scores[np.arange(len(arg)), arg]
    assert np.all(picked >= top[:, 1] - 1e-4 * scale), f"{label}: a pick is not among the best"
    print(f"[parity] {label}: {int(clear.sum())}/{len(arg)} clear, all picks valid", flush=True)


@pytest.mark.parametrize("F,m,d,nv", [
    (100, 64, 32, None),      # one segment, ragged facts
    (1000, 256, 64, None),
    (3000, 512, 128, None),
    (777, 128, 64, 300),      # fewer values than keys: f repeats
])
def test_hebbian_write_read_recall(F, m, d, nv):
    print(f"[case] hebbian F={F} m={m} d={d} nv={nv}", flush=True)
    x = I.draw_facts(F, d, m, seed=F + m + d, n_values=nv)
    K, V, A, G = (dev(x[n]) for n in ("K", "V", "A", "G"))
    f = dev(x["f"])
    Bt = ops.hebbian_write(K, V, f, A, G)
    out = ops.hebbian_read(K, A, G, Bt)
    arg, best = ops.recall_argmax(out[None].contiguous(), V[None].contiguous())
    torch.cuda.synchronize()
    B_ref = Hb.hebbian_write(x["K"], x["V"], x["f"], x["A"], x["G"])
    check("B", Bt.cpu().numpy(), B_ref.T, TOL)
    out_ref = Hb.hebbian_read(x["K"], B_ref, x["A"], x["G"])
    check("read", out.cpu().numpy(), out_ref, TOL)
    check_argmax(arg.cpu().numpy()[0], out_ref, f64(x["V"]), "recall")
    # the stored fraction from the GPU picks agrees with the oracle's within the near-ties
    frac_gpu = float(np.mean(arg.cpu().numpy()[0] == x["f"]))
    frac_ref = Hb.stored_fraction(x["K"], x["V"], x["f"], x["A"], x["G"])
    assert abs(frac_gpu - frac_ref) <= 2.0 / F


def test_hebbian_index_outside_the_values_adds_nothing():
    x = I.draw_facts(200, 32, 64, seed=3)
    f = x["f"].copy()
    f[::7] = -1
    f[3::7] = 1000
    Bt = ops.hebbian_write(dev(x["K"]), dev(x["V"]), dev(f), dev(x["A"]), dev(x["G"]))
    torch.cuda.synchronize()
    keep = (f >= 0) & (f < 200)
    Phi = Hb.features(x["K"], x["A"], x["G"])
    ref = f64(x["V"])[f[keep]].T @ Phi[keep] / 200
    check("B", Bt.cpu().numpy(), ref.T, TOL)


@pytest.mark.parametrize("groups,n,d", [(3, 100, 64), (1, 64, 32), (5, 7, 128), (2, 130, 128)])
def test_memory_read(groups, n, d):
    rng = np.random.default_rng(groups * n + d)
    Q = rng.standard_normal((groups, n, d)).astype(np.float32)
    A = rng.standard_normal((groups, d, d)).astype(np.float32)
    out = ops.tc_memory_read(dev(Q), dev(A))
    torch.cuda.synchronize()
    ref = np.einsum("gni,giv->gnv", f64(Q), f64(A))
    check("q A", out.cpu().numpy(), ref, TOL)


@pytest.mark.parametrize("groups,nq,nc,d", [(4, 70, 1000, 64), (1, 5, 3, 32), (2, 200, 129, 128)])
def test_recall_argmax_groups(groups, nq, nc, d):
    rng = np.random.default_rng(nq + nc)
    R = rng.standard_normal((groups, nq, d)).astype(np.float32)
    V = rng.standard_normal((groups, nc, d)).astype(np.float32)
    arg, best = ops.recall_argmax(dev(R), dev(V))
    torch.cuda.synchronize()
    for gr in range(groups):
        check_argmax(arg.cpu().numpy()[gr], f64(R[gr]), f64(V[gr]), f"group {gr}")
        ref_best = np.max(f64(R[gr]) @ f64(V[gr]).T, axis=1)
        check("best", best.cpu().numpy()[gr], ref_best, TOL)


def test_recall_argmax_ties_take_the_smallest_index():
    V = np.zeros((1, 200, 32), np.float32)
    V[0, :, 0] = 1.0  # every candidate equal
    R = np.zeros((1, 3, 32), np.float32)
    R[0, :, 0] = 1.0
    arg, _ = ops.recall_argmax(dev(R), dev(V))
    torch.cuda.synchronize()
    assert arg.cpu().numpy().tolist() == [[0, 0, 0]]


@pytest.mark.parametrize("tied", [(37, 150, 199), (37, 101, 165), (200, 64, 63), (130, 2)])
def test_recall_argmax_planted_ties(tied):
    # equal maxima in different lanes, in the same lane of different 64-value
    # chunks, and across chunk edges: the smallest index wins
    V = np.full((1, 260, 32), 0.0, np.float32)
    V[0, :, 0] = 0.5
    for j in tied:
        V[0, j, 0] = 1.0
    R = np.zeros((1, 5, 32), np.float32)
    R[0, :, 0] = 1.0
    arg, best = ops.recall_argmax(dev(R), dev(V))
    torch.cuda.synchronize()
    assert arg.cpu().numpy().tolist() == [[min(tied)] * 5]
    assert np.all(best.cpu().numpy() == 1.0)


def test_hebbian_workload_full_size_sampled():
    # F = 16384 facts, m = 4096 features, d = 128: B in full, reads and recall
    # of 512 sampled facts
    w = I.FACT_WORKLOADS["hebbian_f32"]
    print("[case] hebbian full size", flush=True)
    x = I.draw_facts(w.F, w.d, w.m, seed=w.seed)
    K, V, A, G = (dev(x[n]) for n in ("K", "V", "A", "G"))
    Bt = ops.hebbian_write(K, V, dev(x["f"]), A, G)
    rows = np.random.default_rng(0).choice(w.F, 512, replace=False)
    Q = K[torch.from_numpy(rows).cuda()].contiguous()
    out = ops.hebbian_read(Q, A, G, Bt)
    arg, _ = ops.recall_argmax(out[None].contiguous(), V[None].contiguous())
    torch.cuda.synchronize()
    B_ref = Hb.hebbian_write(x["K"], x["V"], x["f"], x["A"], x["G"])
    check("B", Bt.cpu().numpy(), B_ref.T, TOL)
    out_ref = Hb.hebbian_read(x["K"][rows], B_ref, x["A"], x["G"])
    check("read", out.cpu().numpy(), out_ref, TOL)
    check_argmax(arg.cpu().numpy()[0], out_ref, f64(x["V"]), "recall")
