"""The LoRA products of several layers in one launch: qlora_lora_down_batch (t = s x A) and
qlora_lora_u_batch (u = s dy B^T).

"bitsandbytes deep dive" 12.2: the rank-r side path of each layer is t = s x A, and by the
chain rule u = s dy B^T feeds dx and dA.  Each batched output must equal the single-layer
call's bit for bit (qlora_lora_down for t, qlora_linear_bwd_dx for u: the same kernel body,
split plan and summation order); the ragged cases are also checked against the fp64 oracle.
Every output starts out as NaN (tests/conftest.py), so a row that no workgroup writes fails.
"""
import numpy as np
import pytest

from oracle import bf16, lora
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _same(a, b):
    import torch
    return a.shape == b.shape and bool(torch.equal(a, b))


@pytest.mark.parametrize("r", [8, 40, 64])
def test_batched_products_equal_single_calls_and_oracle(q, r):
    import torch
    shapes = [(200, 192), (1000, 4096), (130, 640), (2050, 1152), (0, 256)]
    say(f"[lora batch] t and u on {shapes} r={r}")
    alpha = 2.0 * r
    xs = [workloads.custom(9100 + i, (M, C), 1.0) for i, (M, C) in enumerate(shapes)]
    As = [workloads.custom(9200 + i, (C, r), 1.0 / np.sqrt(r)) for i, (M, C) in enumerate(shapes)]
    Bs = [workloads.custom(9300 + i, (r, C), 0.05) for i, (M, C) in enumerate(shapes)]
    xd, Ad, Bd = [dev_bf16(v) for v in xs], [dev_bf16(v) for v in As], [dev_bf16(v) for v in Bs]
    t_b = q.lora_down_batch(list(zip(xd, Ad)), alpha)
    u_b = q.lora_u_batch(list(zip(xd, Bd)), alpha)
    t_1 = [q.lora_down(x, A, alpha) for x, A in zip(xd, Ad)]
    # u of the single-layer backward: a weight whose rows match B's columns
    u_1 = []
    for x, B, (M, C) in zip(xd, Bd, shapes):
        w = q.quantize(dev_bf16(workloads.custom(9400, (C, 64), 0.02)))
        A64 = dev_bf16(workloads.custom(9401, (64, r), 0.1))
        u_1.append(q.linear_bwd_dx(w, A64, B, alpha, x)[0])
    torch.cuda.synchronize()
    s = lora.lora_scale(alpha, r)
    for i, (M, C) in enumerate(shapes):
        assert _same(t_b[i], t_1[i]), f"item {i}: t differs from qlora_lora_down"
        assert _same(u_b[i], u_1[i]), f"item {i}: u differs from qlora_linear_bwd_dx"
        if M == 0:
            continue
        xf = bf16.to_f64(xs[i])
        et = lora.rel_err(host_f64(t_b[i]), s * (xf @ bf16.to_f64(As[i])))
        eu = lora.rel_err(host_f64(u_b[i]), s * (xf @ bf16.to_f64(Bs[i]).T))
        say(f"    item {i} {M}x{C}: t {et:.2e}, u {eu:.2e}")
        assert et <= 5e-3 and eu <= 5e-3


def test_batched_products_nine_items_two_launches(q):
    import torch
    r, alpha = 16, 32.0
    shapes = [(128 + 40 * i, 64 * (1 + i % 4)) for i in range(9)]
    say(f"[lora batch] nine items {shapes}")
    xd = [dev_bf16(workloads.custom(9500 + i, s_, 1.0)) for i, s_ in enumerate(shapes)]
    Ad = [dev_bf16(workloads.custom(9600 + i, (C, r), 0.25)) for i, (M, C) in enumerate(shapes)]
    t_b = q.lora_down_batch(list(zip(xd, Ad)), alpha)
    t_1 = [q.lora_down(x, A, alpha) for x, A in zip(xd, Ad)]
    torch.cuda.synchronize()
    for i in range(9):
        assert _same(t_b[i], t_1[i]), f"item {i}"


def test_batched_products_7b_block_groups(q):
    """The decoder block's groups that share their input (q/k/v, gate/up) at M = 4096, r = 64."""
    import torch
    wl = workloads.BLOCK_7B
    cfg = workloads.CONFIGS[wl]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    say(f"[lora batch] 7B block groups, M={M} r={r}")
    layers = cfg["layers"]
    for group in ([0, 1, 2], [4, 5]):
        xd = [dev_bf16(workloads.activations(wl, li)) for li in group]
        Ad = [dev_bf16(workloads.lora_A(wl, li)) for li in group]
        Bd = [dev_bf16(workloads.lora_B(wl, li)) for li in group]
        dyd = [dev_bf16(workloads.grad_output(wl, li)) for li in group]
        t_b = q.lora_down_batch(list(zip(xd, Ad)), alpha)
        u_b = q.lora_u_batch(list(zip(dyd, Bd)), alpha)
        for j, li in enumerate(group):
            w = q.quantize(dev_bf16(workloads.weight(wl, li)))
            t_1 = q.lora_down(xd[j], Ad[j], alpha)
            u_1, _ = q.linear_bwd_dx(w, Ad[j], Bd[j], alpha, dyd[j])
            torch.cuda.synchronize()
            assert _same(t_b[j], t_1), f"{layers[li][0]}: t differs"
            assert _same(u_b[j], u_1), f"{layers[li][0]}: u differs"
            assert bool(torch.isfinite(t_b[j].float()).all()) and bool(torch.isfinite(u_b[j].float()).all())
            say(f"    {layers[li][0]}: equal")
