"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): a serving
loop captures one decode step (and the caller's position advance) once and
replays it per token; a prefill captures one fused-layer, scan or delta-rule
call (with the workspace the wrapper allocates inside the capture).  Every replay
is checked against the same call made eagerly: the kernels use no atomics,
so the results must agree bit for bit.  Eager work (input copies, other
calls, synchronisations) runs between the replays."""
import numpy as np
import pytest
import torch

from linear_attention_tensor_amd import inputs as I
from linear_attention_tensor_amd import ops
from tests._helpers import f32_dev, to_dev

pytestmark = pytest.mark.gpu


def _decode_case(B, H, d, W, S, seed):
    x = I.draw(B, H, S, d, seed=seed, dtype="bf16")
    q = to_dev(x["q"], "bf16").permute(2, 0, 1, 3).contiguous()  # [S, B, H, d]
    k = to_dev(x["k"], "bf16").permute(2, 0, 1, 3).contiguous()
    v = to_dev(x["v"], "bf16").permute(2, 0, 1, 3).contiguous()
    rk, rv = I.draw_ring(B, H, W, d, seed=seed + 1)
    sc = I.decode_scalars(H, seed=seed + 2)
    g = torch.tensor(np.random.default_rng(seed + 3).standard_normal(H), dtype=torch.float32, device="cuda")
    return q, k, v, to_dev(rk, "bf16"), to_dev(rv, "bf16"), f32_dev(sc["lam"]), f32_dev(sc["eta"]), g


@pytest.mark.parametrize("layer", [False, True], ids=["l2_step", "layer_step"])
def test_decode_step_graph_replays(layer):
    B, H, d, W, S = 2, 3, 64, 16, 40
    print(f"[case] decode graph layer={layer} B={B} H={H} d={d} W={W} steps={S}", flush=True)
    q, k, v, rk0, rv0, lam, eta, g = _decode_case(B, H, d, W, S, seed=321)
    A0 = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    pos0 = torch.tensor([0, 5], dtype=torch.int64, device="cuda")  # one ring still filling

    def step(qi, ki, vi, rk, rv, A, pos, out):
        if layer:
            return ops.tc_decode_layer_step(qi, ki, vi, rk, rv, A, lam, eta, g, pos, W, y=out, check_values=False)
        return ops.tc_decode_step(qi, ki, vi, rk, rv, A, lam, eta, pos, W, m=out, check_values=False)

    # eager reference
    rk, rv, A, pos = rk0.clone(), rv0.clone(), A0.clone(), pos0.clone()
    ref = []
    for t in range(S):
        ref.append(step(q[t], k[t], v[t], rk, rv, A, pos, None).clone())
        pos += 1
    torch.cuda.synchronize()
    ref_state = (rk, rv, A, pos)

    # one captured step on static buffers, with the position advance
    qs, ks, vs = q[0].clone(), k[0].clone(), v[0].clone()
    grk, grv, gA, gpos = rk0.clone(), rv0.clone(), A0.clone(), pos0.clone()
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(qs, ks, vs, grk, grv, gA, gpos, out)
        gpos += 1
    torch.cuda.synchronize()
    for rnd in range(2):  # the same token stream twice, from the same start
        grk.copy_(rk0)
        grv.copy_(rv0)
        gA.copy_(A0)
        gpos.copy_(pos0)
        for t in range(S):
            qs.copy_(q[t])
            ks.copy_(k[t])
            vs.copy_(v[t])
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref[t]), f"round {rnd} step {t}"
        for got, want in zip((grk, grv, gA, gpos), ref_state):
            assert torch.equal(got, want), f"round {rnd} state"


def test_fused_layer_graph_replays():
    B, H, T, d, W = 1, 2, 700, 64, 100
    print(f"[case] fused graph B={B} H={H} T={T} d={d} W={W}", flush=True)
    xs = [I.draw(B, H, T, d, seed=900 + i, dtype="bf16", lam=("uniform", 0.95, 0.999)) for i in range(3)]
    g = torch.tensor([0.3, -1.2], dtype=torch.float32, device="cuda")

    def inputs(x):
        return (to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                f32_dev(x["lam"]), f32_dev(x["eta"]))

    refs = []
    for x in xs:
        qi, ki, vi, lam, eta = inputs(x)
        y, A = ops.tc_fused_layer(qi, ki, vi, lam, eta, g, W, return_state=True)
        refs.append((y.clone(), A.clone()))
    torch.cuda.synchronize()

    qs, ks, vs, lams, etas = (t.clone() for t in inputs(xs[0]))
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        ys, As = ops.tc_fused_layer(qs, ks, vs, lams, etas, g, W, return_state=True, check_values=False)
    torch.cuda.synchronize()
    for rnd, i in enumerate([0, 1, 2, 0, 2]):
        qi, ki, vi, lam, eta = inputs(xs[i])
        for dst, src in ((qs, qi), (ks, ki), (vs, vi), (lams, lam), (etas, eta)):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, refs[i][0]), f"replay {rnd} (input {i}): y"
        assert torch.equal(As, refs[i][1]), f"replay {rnd} (input {i}): A"
        # eager work between replays: the layer on another input
        j = (i + 1) % 3
        qj, kj, vj, lj, ej = inputs(xs[j])
        assert torch.equal(ops.tc_fused_layer(qj, kj, vj, lj, ej, g, W), refs[j][0])


def _graph_vs_eager(call, make_inputs, n_inputs, what):
    """Capture call(*static) once, replay it on several inputs copied into the
    static tensors (eager calls between the replays) and compare every output
    with the eager call on the same input, bit for bit."""
    ins = [make_inputs(i) for i in range(n_inputs)]
    refs = [tuple(t.clone() for t in call(*x)) for x in ins]
    torch.cuda.synchronize()
    static = tuple(t.clone() for t in ins[0])
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        outs = call(*static)
    torch.cuda.synchronize()
    for rnd, i in enumerate([1, 0, n_inputs - 1, 1]):
        for dst, src in zip(static, ins[i]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        for j, (got, want) in enumerate(zip(outs, refs[i])):
            assert torch.equal(got, want), f"{what}: replay {rnd} (input {i}), output {j}"
        other = ins[(i + 1) % n_inputs]  # eager work between the replays
        assert all(torch.equal(a, b) for a, b in zip(call(*other), refs[(i + 1) % n_inputs]))


@pytest.mark.parametrize("dtype,d,T,W", [("f32", 64, 900, 100), ("bf16", 128, 1500, 256), ("bf16", 32, 300, 40)])
def test_scan_forward_graph_replays(dtype, d, T, W):
    print(f"[case] scan graph dtype={dtype} d={d} T={T} W={W}", flush=True)

    def make(i):
        x = I.draw(1, 3, T, d, seed=950 + i, dtype=dtype, lam=("uniform", 0.95, 0.999))
        return (to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype), f32_dev(x["lam"]),
                f32_dev(x["eta"]))

    def call(q, k, v, lam, eta):
        return ops.tc_scan_forward(q, k, v, lam, eta, W, check_values=False)

    _graph_vs_eager(call, make, 3, "tc_scan_forward")


@pytest.mark.parametrize("dtype,d,T", [("f32", 64, 700), ("bf16", 128, 600)])
def test_delta_forward_graph_replays(dtype, d, T):
    print(f"[case] delta graph dtype={dtype} d={d} T={T}", flush=True)

    def make(i):
        x = I.draw(1, 2, T, d, seed=970 + i, dtype=dtype)
        rng = np.random.default_rng(980 + i)
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, 2, T))))
        return (to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype), f32_dev(beta))

    def call(q, k, v, beta):
        return ops.delta_scan_forward(q, k, v, beta, return_state=True, check_values=False)

    _graph_vs_eager(call, make, 3, "delta_scan_forward")
