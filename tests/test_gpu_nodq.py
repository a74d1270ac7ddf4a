"""Parity of the path without double quantization (fp32 block absmax, 4.5
bits/param; "bitsandbytes deep dive" 7.1 and 9.5) with the CPU oracle.

Bars: packed codes, the fp32 absmax and the dequantized bf16 weight
bit-exact; y, t, dx, dA, dB within 5e-3 normwise relative error (bf16
inputs, fp32 accumulation).  The shapes walk the GEMM's even and odd block
counts per row, a single super-step, ragged M/N/r, and the decode GEMV.
"""
import numpy as np
import pytest

from oracle import bf16, lora, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


@pytest.mark.parametrize("N,K", [(256, 256), (4096, 4096), (3, 192), (257, 64), (64, 11008)])
def test_quantize_dequantize_bit_exact(q, N, K):
    import torch
    W = workloads.weight(workloads.Q_PROJ_DECODE) if (N, K) == (4096, 4096) else workloads.custom(300 + N + K, (N, K), 0.02)
    say(f"[nodq quantize] N={N} K={K}")
    w = q.quantize(dev_bf16(W), double_quant=False)
    assert w.q8 is None and w.a2.numel() == N * K // 64
    wh = q.dequantize(w)
    torch.cuda.synchronize()
    rc, ra = nf4.quantize_nodq(W)
    assert np.array_equal(w.codes.cpu().numpy(), rc)
    assert np.array_equal(w.a2.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(host_bits(wh), nf4.dequantize_nodq(rc, ra, N, K))


def _check_linear(q, M, N, K, r, seed, alpha):
    import torch
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    say(f"[nodq linear] M={M} N={N} K={K} r={r}")
    w = q.quantize(dev_bf16(W), double_quant=False)
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    dx, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t)
    torch.cuda.synchronize()
    p, a = nf4.quantize_nodq(W)
    Wh = bf16.to_f64(nf4.dequantize_nodq(p, a, N, K))
    xf, Af, Bf, dyf = (bf16.to_f64(v) for v in (x, A, B, dy))
    ry, rt = lora.linear_fwd(xf, Wh, Af, Bf, alpha, r)
    rdx, rdA, rdB = lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
    errs = {k: lora.rel_err(host_f64(g), ref) for k, g, ref in
            (("y", y, ry), ("t", t, rt), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB))}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{k} rel err {e:.3e}"


@pytest.mark.parametrize("M,N,K,r", [
    (256, 256, 256, 8),          # the 256 x 256 single-linear size
    (17, 130, 128, 8),           # one super-step of two blocks
    (300, 520, 384, 64),         # ragged M and N
    (64, 72, 11008 // 4, 32),    # 43 blocks per row: odd count, short last super-step
    (257, 256, 256, 100),        # r > 96
])
def test_linear(q, M, N, K, r):
    _check_linear(q, M, N, K, r, 500 + M + N + K + r, 2.0 * r)


@pytest.mark.parametrize("M,N,K,r", [(1, 4096, 4096, 16), (16, 4096, 4096, 16), (5, 33, 4160, 128)])
def test_decode_gemv(q, M, N, K, r):
    import torch
    seed = 900 + M + r
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    say(f"[nodq gemv] M={M} N={N} K={K} r={r}")
    w = q.quantize(dev_bf16(W), double_quant=False)
    y, t = q.linear_fwd(w, dev_bf16(x), dev_bf16(A), dev_bf16(B), 2.0 * r)
    torch.cuda.synchronize()
    p, a = nf4.quantize_nodq(W)
    Wh = bf16.to_f64(nf4.dequantize_nodq(p, a, N, K))
    ry, rt = lora.linear_fwd(bf16.to_f64(x), Wh, bf16.to_f64(A), bf16.to_f64(B), 2.0 * r, r)
    ey, et = lora.rel_err(host_f64(y), ry), lora.rel_err(host_f64(t), rt)
    say(f"    rel err y {ey:.3e}  t {et:.3e}")
    assert ey <= TOL and et <= TOL
