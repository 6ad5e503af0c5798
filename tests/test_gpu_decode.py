"""Parity of tc_decode_step (C ABI, HIP kernel) against the float64 oracle."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from oracle import tc as O
from tests._helpers import f32_dev, check, report, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,d,W,T", [(2, 3, 64, 8, 40), (1, 2, 128, 5, 23), (3, 1, 16, 1, 9), (1, 1, 32, 64, 70)])
def test_decode_from_empty_matches_scan(dtype, B, H, d, W, T):
    print(f"[case] decode dtype={dtype} B={B} H={H} d={d} W={W} T={T}", flush=True)
    x = I.draw(B, H, T, d, seed=300 + d + W, dtype=dtype)
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"], W)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ring_k = torch.zeros((B, H, W, d), dtype=tdt, device="cuda")
    ring_v = torch.zeros((B, H, W, d), dtype=tdt, device="cuda")
    A = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    lam, eta = f32_dev(x["lam"]), f32_dev(x["eta"])
    ms = []
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        ms.append(ops.tc_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                     ring_k, ring_v, A, lam, eta, pos, W).clone())
    m = torch.stack(ms, dim=2).cpu().numpy()
    check("m", m, m_ref, TOL[dtype])
    check("A", A.cpu().numpy(), A_ref, TOL[dtype])
    # the ring holds the last W tokens in slots t mod W, bit for bit
    rk = ring_k.cpu()
    kk = k.cpu()
    for t in range(max(0, T - W), T):
        assert torch.equal(rk[:, :, t % W], kk[:, :, t])


def test_decode_sequences_at_different_positions():
    B, H, d, W = 3, 2, 64, 6
    rng = np.random.default_rng(9)
    pos0 = np.array([0, 4, 17])
    ring_k = rng.standard_normal((B, H, W, d)).astype(np.float32)
    ring_v = rng.standard_normal((B, H, W, d)).astype(np.float32)
    A0 = (rng.standard_normal((B, H, d, d)) * 0.1).astype(np.float32)
    sc = I.decode_scalars(H)
    dec = O.TensorCacheDecoder.from_state(ring_k.astype(np.float64), ring_v.astype(np.float64),
                                          A0.astype(np.float64), pos0, W, sc["lam"], sc["eta"])
    g_rk, g_rv, g_A = f32_dev(ring_k), f32_dev(ring_v), f32_dev(A0)
    lam, eta = f32_dev(sc["lam"]), f32_dev(sc["eta"])
    for step in range(12):
        x = I.draw_decode_position(B, H, d, 1000 + step, dtype="f32")
        pos = torch.from_numpy(pos0 + step).to("cuda")
        m = ops.tc_decode_step(to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
                               g_rk, g_rv, g_A, lam, eta, pos, W)
        m_ref = dec.step(x["q64"], x["k64"], x["v64"])
        check(f"step {step}", m.cpu().numpy(), m_ref, 1e-5)
    check("A", g_A.cpu().numpy(), dec.A, 1e-5)


def test_scan_prefill_then_decode_continues_the_scan():
    # prefill T0 tokens with the scan, hand over A_final and the last W tokens,
    # decode the rest: every decoded read and the final A against the oracle's
    # scan of the whole sequence (the bf16 bar), and against the GPU scan of the
    # whole sequence (bf16 scans round P and the state to bf16 for the MFMAs)
    B, H, d, W, T0, T = 1, 2, 128, 16, 100, 130
    x = I.draw(B, H, T, d, seed=55, dtype="bf16")
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    lam, eta = f32_dev(x["lam"]), f32_dev(x["eta"])
    m_ref, A_ref = O.tc_scan(x["q64"], x["k64"], x["v64"], x["lam"].astype(np.float64), x["eta"], W)
    m_full, A_full = ops.tc_scan_forward(q, k, v, lam, eta, W)
    _, A = ops.tc_scan_forward(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(),
                               v[:, :, :T0].contiguous(), lam, eta, W)
    ring_k = torch.empty((B, H, W, d), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.empty_like(ring_k)
    for t in range(T0 - W, T0):
        ring_k[:, :, t % W] = k[:, :, t]
        ring_v[:, :, t % W] = v[:, :, t]
    for t in range(T0, T):
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        m = ops.tc_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                               ring_k, ring_v, A, lam, eta, pos, W)
        check(f"t={t}", m.cpu().numpy(), m_ref[:, :, t], 2e-2)
        check(f"t={t} vs GPU scan", m.cpu().numpy(), m_full[:, :, t].cpu().numpy(), 1e-2)
    check("A", A.cpu().numpy(), A_ref, 2e-2)
    check("A vs GPU scan", A.cpu().numpy(), A_full.cpu().numpy(), 1e-2)


def test_decode_workload_full_size_sampled_sequences():
    # 64 sequences x 32 heads, d = 128, W = 2048, bf16, full ring at pos = W, A = 0
    w = I.WORKLOADS["decode_bf16"]
    B, H, d, W = w.B, w.H, w.d, w.W
    print("[case] decode full size", flush=True)
    rk, rv = I.draw_ring(B, H, W, d)
    sc = I.decode_scalars(H)
    g_rk, g_rv = to_dev(rk, "bf16"), to_dev(rv, "bf16")
    g_A = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    lam, eta = f32_dev(sc["lam"]), f32_dev(sc["eta"])
    bs = [0, 13, 63]
    dec = O.TensorCacheDecoder.from_state(I.storage_to_f64(rk[bs], "bf16"), I.storage_to_f64(rv[bs], "bf16"),
                                          np.zeros((len(bs), H, d, d)), np.full(len(bs), W), W,
                                          sc["lam"], sc["eta"])
    for step in range(6):
        x = I.draw_decode_position(B, H, d, W + step)
        pos = torch.full((B,), W + step, dtype=torch.int64, device="cuda")
        m = ops.tc_decode_step(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                               g_rk, g_rv, g_A, lam, eta, pos, W)
        m_ref = dec.step(x["q64"][bs], x["k64"][bs], x["v64"][bs])
        check(f"step {step}", m.cpu().numpy()[bs], m_ref, 2e-2)
    check("A", g_A.cpu().numpy()[bs], dec.A, 2e-2)
