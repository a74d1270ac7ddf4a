"""The backward with deferred LoRA weight gradients: qlora_linear_bwd_dx per layer, then
qlora_lora_grads_batch over all layers in one launch.

With the base weight frozen ("bitsandbytes deep dive" 12.4) only the LoRA factors get
gradients; dA = x^T u and dB = t^T dy are needed by the optimizer step alone, so a
backward pass may compute them after every layer's dx.  The split calls run the same
kernels with the same split plans as qlora_linear_bwd, so u, dx, dA and dB must equal its
outputs bit for bit; the small cases are also checked against the fp64 oracle (12.2: the
chain rule through Y = XW + s X A B).  Every output starts out as NaN (tests/conftest.py),
so an element that no workgroup writes fails.
"""
import numpy as np
import pytest

from oracle import bf16, lora, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _layer(q, seed, M, N, K, r):
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), 1.0 / np.sqrt(r))
    B = workloads.custom(seed + 3, (r, N), 0.05)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    host = dict(W=W, x=x, A=A, B=B, dy=dy)
    d = dict(w=q.quantize(dev_bf16(W)), x=dev_bf16(x), A=dev_bf16(A), B=dev_bf16(B), dy=dev_bf16(dy), M=M, N=N,
             K=K)
    return host, d


def _run(q, layers, alpha):
    """The layer backward both ways: qlora_linear_bwd per layer, and the split calls."""
    import torch
    ref, got_u, got_dx = [], [], []
    for d in layers:
        _, d["t"] = q.linear_fwd(d["w"], d["x"], d["A"], d["B"], alpha)
        ref.append(q.linear_bwd(d["w"], d["x"], d["A"], d["B"], alpha, d["dy"], t=d["t"]))
    for d in layers:
        u, dx = q.linear_bwd_dx(d["w"], d["A"], d["B"], alpha, d["dy"])
        got_u.append(u)
        got_dx.append(dx)
    dA, dB = q.lora_grads_batch([(d["x"], d["t"], u, d["dy"]) for d, u in zip(layers, got_u)])
    torch.cuda.synchronize()
    return ref, got_u, got_dx, dA, dB


def _same(a, b):
    import torch
    return a.shape == b.shape and bool(torch.equal(a, b))


SHAPES = [(200, 72, 192), (256, 520, 128), (1000, 1152, 256), (130, 64, 640)]


@pytest.mark.parametrize("r", [24, 64])
def test_deferred_equals_linear_bwd_and_oracle(q, r):
    say(f"[deferred grads] ragged layers {SHAPES} r={r}")
    alpha = 16.0
    pairs = [_layer(q, 8100 + 10 * i + r, M, N, K, r) for i, (M, N, K) in enumerate(SHAPES)]
    layers = [d for _, d in pairs]
    ref, us, dxs, dA, dB = _run(q, layers, alpha)
    for i, ((h, d), (dx_r, dA_r, dB_r)) in enumerate(zip(pairs, ref)):
        assert _same(dxs[i], dx_r), f"layer {i}: dx differs from qlora_linear_bwd"
        assert _same(dA[i], dA_r), f"layer {i}: dA differs from qlora_linear_bwd"
        assert _same(dB[i], dB_r), f"layer {i}: dB differs from qlora_linear_bwd"
        N, K = d["N"], d["K"]
        xf, Af, Bf, dyf = (bf16.to_f64(h[k]) for k in ("x", "A", "B", "dy"))
        p, q8, a2 = nf4.quantize(h["W"])
        Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
        dx_o, dA_o, dB_o = lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
        u_o = lora.lora_scale(alpha, r) * (dyf @ Bf.T)
        errs = dict(u=lora.rel_err(host_f64(us[i]), u_o), dx=lora.rel_err(host_f64(dxs[i]), dx_o),
                    dA=lora.rel_err(host_f64(dA[i]), dA_o), dB=lora.rel_err(host_f64(dB[i]), dB_o))
        say(f"    layer {i} {d['M']}x{N}x{K}: rel errors {errs}")
        for k, e in errs.items():
            assert e <= 5e-3, f"layer {i} {k}: {e:.3e}"


def test_deferred_nine_layers_two_launches_and_empty(q):
    """Nine layers take two launches (at most 8 layers per launch); an empty layer gets zero gradients."""
    import torch
    r, alpha = 16, 32.0
    shapes = [(136 + 8 * i, 64 * (1 + i % 3), 128 + 64 * (i % 2)) for i in range(8)] + [(0, 200, 192)]
    say(f"[deferred grads] nine layers {shapes} r={r}")
    layers = [_layer(q, 8300 + 10 * i, M, N, K, r)[1] for i, (M, N, K) in enumerate(shapes)]
    ref, us, dxs, dA, dB = _run(q, layers, alpha)
    for i, (dx_r, dA_r, dB_r) in enumerate(ref):
        assert _same(dA[i], dA_r) and _same(dB[i], dB_r), f"layer {i}: gradients differ from qlora_linear_bwd"
        if layers[i]["M"]:
            assert _same(dxs[i], dx_r), f"layer {i}: dx differs"
    assert float(dA[8].abs().max()) == 0.0 and float(dB[8].abs().max()) == 0.0
    assert not bool(torch.isnan(dA[8]).any())


def test_deferred_7b_block_bench_shapes(q):
    """The decoder block the benchmark times (7 linears, M = 4096 tokens, r = 64): u, dx, dA and dB of
    the split calls equal qlora_linear_bwd's bit for bit (whose outputs the full-size parity tests check
    against the oracle) and are finite."""
    import torch
    wl = workloads.BLOCK_7B
    cfg = workloads.CONFIGS[wl]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    say(f"[deferred grads] 7B block, M={M} r={r}")
    layers = []
    for li, (name, N, K) in enumerate(cfg["layers"]):
        layers.append(dict(w=q.quantize(dev_bf16(workloads.weight(wl, li))), x=dev_bf16(workloads.activations(wl, li)),
                           A=dev_bf16(workloads.lora_A(wl, li)), B=dev_bf16(workloads.lora_B(wl, li)),
                           dy=dev_bf16(workloads.grad_output(wl, li)), M=M, N=N, K=K))
    ref, us, dxs, dA, dB = _run(q, layers, alpha)
    for i, (dx_r, dA_r, dB_r) in enumerate(ref):
        name = cfg["layers"][i][0]
        assert _same(dxs[i], dx_r), f"{name}: dx differs from qlora_linear_bwd"
        assert _same(dA[i], dA_r), f"{name}: dA differs from qlora_linear_bwd"
        assert _same(dB[i], dB_r), f"{name}: dB differs from qlora_linear_bwd"
        for k, v in (("u", us[i]), ("dA", dA[i]), ("dB", dB[i])):
            assert bool(torch.isfinite(v).all()), f"{name}: {k} not finite"
        say(f"    {name}: equal")
