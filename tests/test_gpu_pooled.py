"""Parity of the QA-LoRA pooled branch (qlora_pooled_fwd / qlora_pooled_bwd;
"LoRA, QLoRA, QA-LoRA explained", sections 3-5) with the fp64 oracle.

Bar: y, t, dx, dA [K/g, r], dB within 5e-3 normwise relative error.  g runs
over the NF4 block (64), smaller groups (32, 2), ragged shapes, and g = 1,
which must equal the plain layer bit for bit (the pooled path runs the same
kernels on A~ = A).
"""
import numpy as np
import pytest

from oracle import bf16, lora, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


@pytest.mark.parametrize("M,N,K,r,g", [(256, 256, 256, 8, 64), (300, 520, 384, 64, 32), (17, 130, 128, 8, 2),
                                       (64, 72, 2752, 16, 64), (8, 4096, 4096, 16, 64)])
def test_pooled_fwd_bwd(q, M, N, K, r, g):
    import torch
    seed = 1100 + M + N + K + r + g
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K // g, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[pooled] M={M} N={N} K={K} r={r} g={g}")
    w = q.quantize(dev_bf16(W))
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.pooled_fwd(w, xd, Ad, Bd, alpha, g)
    dx, dA, dB = q.pooled_bwd(w, xd, Ad, Bd, alpha, g, dyd, t=t)
    torch.cuda.synchronize()
    p, q8, a2 = nf4.quantize(W)
    Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
    xf, Af, Bf, dyf = (bf16.to_f64(v) for v in (x, A, B, dy))
    ry, rt = lora.pooled_fwd(xf, Wh, Af, Bf, alpha, r, g)
    rdx, rdA, rdB = lora.pooled_bwd(xf, Wh, Af, Bf, alpha, r, g, dyf)
    errs = {k: lora.rel_err(host_f64(v), ref) for k, v, ref in
            (("y", y, ry), ("t", t, rt), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB))}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{k} rel err {e:.3e}"


def test_group_one_equals_plain_layer(q):
    import torch
    M, N, K, r = 64, 192, 256, 16
    W = workloads.custom(1201, (N, K), 0.02)
    x, A, B, dy = (dev_bf16(workloads.custom(1202 + i, s, v)) for i, (s, v) in
                   enumerate((((M, K), 1.0), ((K, r), 0.25), ((r, N), 0.01), ((M, N), 1.0))))
    w = q.quantize(dev_bf16(W))
    y1, t1 = q.pooled_fwd(w, x, A, B, 32.0, 1)
    g1 = q.pooled_bwd(w, x, A, B, 32.0, 1, dy, t=t1)
    y2, t2 = q.linear_fwd(w, x, A, B, 32.0)
    g2 = q.linear_bwd(w, x, A, B, 32.0, dy, t=t2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))
