"""Seeded input generator: determinism, distribution, and bf16 rounding."""
import numpy as np
import torch

from linear_attention_tensor_amd import inputs as I


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1 + 2**-8, 1 + 3 * 2**-9, 3.0e38, -1e-40], np.float32)])
    ours = I.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(I.bf16_bits_to_f64(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_draw_is_deterministic_and_keys_are_unit():
    a = I.draw(2, 3, 50, 16, seed=7, dtype="bf16")
    b = I.draw(2, 3, 50, 16, seed=7, dtype="bf16")
    for n in ("q", "k", "v", "lam", "eta", "g", "beta"):
        np.testing.assert_array_equal(a[n], b[n])
    kn = np.linalg.norm(I.draw(2, 3, 50, 16, seed=7, dtype="f32")["k64"], axis=-1)
    np.testing.assert_allclose(kn, 1.0, rtol=1e-6)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_workload_scalars_in_range():
    w = I.WORKLOADS["fused_layer_bf16"]
    x = I.draw(1, w.H, 8, w.d, seed=w.seed, dtype=w.dtype, lam=w.lam, eta=w.eta)
    assert np.all((x["lam"] >= 0.95) & (x["lam"] <= 0.999))
    assert np.all((x["eta"] >= 0.1) & (x["eta"] <= 1.0))
