"""Parity of the LoRA down-projections at training-size M with the fp64 CPU oracle.

t = s x A and u = s dy B^T ("bitsandbytes deep dive" 12.2: the rank-r side
path of the layer and its chain rule) at M >= 2048 rows, checked in full: t
from qlora_lora_down (bf16 and fp16), and u through dA = x^T u of
qlora_linear_bwd.  The shapes take the split reduction through its edge
cases: row counts that are not a multiple of the 128-row panel, reductions
split 2 to 22 ways (the last split partial at K = 11008), and r of 16 to 64
(one to two 32-column tiles, one of them partial at r = 16 and 48).  Every output
starts out as NaN (tests/conftest.py), so a row that no workgroup writes fails.
"""
import numpy as np
import pytest

from oracle import bf16, f16, lora, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, dev_f16, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


@pytest.mark.parametrize("M,K,r", [(2048, 4096, 64), (2056, 1152, 16), (2051, 1152, 48), (4096, 11008, 64),
                                   (2064, 256, 32)])
def test_lora_down_rows_bf16(q, M, K, r):
    import torch
    say(f"[lora rows] t bf16 M={M} K={K} r={r}")
    x = workloads.custom(7100 + r, (M, K), 1.0)
    A = workloads.custom(7200 + r, (K, r), 1.0 / np.sqrt(r))
    alpha = 2.0 * r
    t = q.lora_down(dev_bf16(x), dev_bf16(A), alpha)
    torch.cuda.synchronize()
    ref = lora.lora_scale(alpha, r) * (bf16.to_f64(x) @ bf16.to_f64(A))
    e = lora.rel_err(host_f64(t), ref)
    say(f"    rel error {e:.3e}")
    assert e <= 5e-3


@pytest.mark.parametrize("M,K,r", [(2056, 1152, 64), (2048, 4096, 16)])
def test_lora_down_rows_f16(q, M, K, r):
    import torch
    say(f"[lora rows] t fp16 M={M} K={K} r={r}")
    x = workloads.normal_f16(7300 + r, (M, K), 1.0)
    A = workloads.normal_f16(7400 + r, (K, r), 1.0 / np.sqrt(r))
    alpha = 2.0 * r
    t = q.lora_down(dev_f16(x), dev_f16(A), alpha)
    torch.cuda.synchronize()
    ref = lora.lora_scale(alpha, r) * (f16.to_f64(x) @ f16.to_f64(A))
    e = lora.rel_err(host_f64(t), ref)
    say(f"    rel error {e:.3e}")
    assert e <= 1e-3


@pytest.mark.parametrize("M,N,K,r", [(2056, 1152, 256, 48), (2048, 4096, 128, 64)])
def test_u_rows_through_dA(q, M, N, K, r):
    import torch
    say(f"[lora rows] u via dA M={M} N={N} K={K} r={r}")
    W = workloads.custom(7500, (N, K), 0.02)
    x = workloads.custom(7501, (M, K), 1.0)
    A = workloads.custom(7502, (K, r), 1.0 / np.sqrt(r))
    B = workloads.custom(7503, (r, N), 0.05)
    dy = workloads.custom(7504, (M, N), 1.0)
    alpha = 16.0
    w = q.quantize(dev_bf16(W))
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    _, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t, need_dx=False)
    torch.cuda.synchronize()
    dA_ref, dB_ref = lora.lora_grads(bf16.to_f64(x), bf16.to_f64(A), bf16.to_f64(B), alpha, r, bf16.to_f64(dy))
    p, q8, a2 = nf4.quantize(W)
    y_ref, t_ref = lora.linear_fwd(bf16.to_f64(x), bf16.to_f64(nf4.dequantize(p, q8, a2, N, K)), bf16.to_f64(A),
                                   bf16.to_f64(B), alpha, r)
    errs = dict(dA=lora.rel_err(host_f64(dA), dA_ref), dB=lora.rel_err(host_f64(dB), dB_ref),
                t=lora.rel_err(host_f64(t), t_ref), y=lora.rel_err(host_f64(y), y_ref))
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= 5e-3, f"{k}: {e:.3e}"
