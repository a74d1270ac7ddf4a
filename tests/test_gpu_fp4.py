"""Parity of the fp4 quant type ("bitsandbytes deep dive" 6.5, 8.1; E2M1 levels / 6)
through every entry point that reads or writes codes, against the CPU oracle
(oracle.fp4).

Bar: codes, q8, a2 (or the fp32 absmax without double quantization), the
dequantized weight and the merged weight bit-exact; y, t, dx, dA, dB of the
layer within 5e-3 normwise relative error of the fp64 oracle on the FP4
reconstruction.  Covers the tiled GEMMs (even and odd block counts), the
decode GEMV (M = 1, 16), ragged shapes, both scale layouts, and edge blocks.
"""
import numpy as np
import pytest

from oracle import bf16, fp4, lora, merge, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _quant_check(q, W, dq, tag):
    import torch
    N, K = W.shape
    say(f"[fp4 quantize] {tag} N={N} K={K} double_quant={dq}")
    w = q.quantize(dev_bf16(W), double_quant=dq, quant_type="fp4")
    wh = q.dequantize(w)
    torch.cuda.synchronize()
    codes = w.codes.cpu().numpy()
    if dq:
        rc, rq, ra = fp4.quantize(W)
        assert np.array_equal(w.q8.cpu().numpy(), rq), f"{tag}: q8"
        assert np.array_equal(w.a2.cpu().numpy().view(np.uint32), ra.view(np.uint32)), f"{tag}: a2"
        rwh = fp4.dequantize(rc, rq, ra, N, K)
    else:
        rc, ra = fp4.quantize_nodq(W)
        assert np.array_equal(w.a2.cpu().numpy().view(np.uint32), ra.view(np.uint32)), f"{tag}: absmax"
        rwh = fp4.dequantize_nodq(rc, ra, N, K)
    assert np.array_equal(codes, rc), f"{tag}: codes differ at {np.flatnonzero(codes != rc)[:8]}"
    got = host_bits(wh)
    assert np.array_equal(got, rwh), f"{tag}: dequant differs at {np.flatnonzero(got != rwh)[:8]}"
    return w, rwh


@pytest.mark.parametrize("N,K,dq", [(256, 256, True), (3, 192, True), (257, 64, True), (64, 11008, True),
                                    (5, 640, False), (130, 192, False)])
def test_quantize_dequantize(q, N, K, dq):
    _quant_check(q, workloads.custom(3100 + N + K, (N, K), 0.02), dq, f"{N}x{K}")


def test_edge_blocks(q):
    """All-zero block, blocks of +-0, absmax with both signs, weights exactly on the exact levels
    (0, 1/4, 1/2, 1 times a power of two), subnormal and huge blocks."""
    rng = np.random.default_rng(4321)
    K = 64 * 8
    r0 = rng.standard_normal(K).astype(np.float32) * 0.02
    r0[0:64] = 0.0
    r0[64:128] = -0.0
    r0[128 + 5], r0[128 + 9] = 0.5, -0.5
    r0[192:199] = np.array([0.0, 0.25, 0.5, 1.0, -0.25, -0.5, -1.0], np.float32) * 8.0
    r0[256:320] = (rng.standard_normal(64) * 1e-39).astype(np.float32)
    r0[320:384] = (rng.standard_normal(64) * 1e36).astype(np.float32)
    W = np.concatenate([r0[None, :], bf16.to_f32(workloads.custom(56, (40, K), 0.02))], axis=0)
    W = bf16.from_f32_rne(W)
    w, _ = _quant_check(q, W, True, "edge blocks")
    codes = nf4.unpack_nibbles(w.codes.cpu().numpy())
    assert np.all(codes[0:128] == 0)                        # zeros of either sign encode as +0
    assert not np.any(codes == 8)                           # -0 is never produced
    _quant_check(q, W, False, "edge blocks, no double quantization")


def _layer(q, M, N, K, r, dq, seed, check_dx=True):
    import torch
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[fp4 linear] M={M} N={N} K={K} r={r} double_quant={dq}")
    w = q.quantize(dev_bf16(W), double_quant=dq, quant_type="fp4")
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    dx, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t, need_dx=check_dx)
    torch.cuda.synchronize()
    if dq:
        p, q8, a2 = fp4.quantize(W)
        Wh = bf16.to_f64(fp4.dequantize(p, q8, a2, N, K))
    else:
        p, a = fp4.quantize_nodq(W)
        Wh = bf16.to_f64(fp4.dequantize_nodq(p, a, N, K))
    xf, Af, Bf, dyf = (bf16.to_f64(v) for v in (x, A, B, dy))
    ry, rt = lora.linear_fwd(xf, Wh, Af, Bf, alpha, r)
    rdx, rdA, rdB = lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
    pairs = [("y", y, ry), ("t", t, rt), ("dA", dA, rdA), ("dB", dB, rdB)]
    if check_dx:
        pairs.append(("dx", dx, rdx))
    errs = {k: lora.rel_err(host_f64(v), ref) for k, v, ref in pairs}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{k} rel err {e:.3e}"


@pytest.mark.parametrize("M,N,K,r,dq", [(64, 256, 512, 16, True), (300, 520, 384, 64, True),
                                        (64, 72, 64 * 43, 16, True), (17, 130, 128, 8, False),
                                        (257, 256, 256, 100, False)])
def test_linear_tiled(q, M, N, K, r, dq):
    _layer(q, M, N, K, r, dq, 3200 + M + N + K + r)


@pytest.mark.parametrize("M,dq", [(1, True), (16, True), (1, False), (5, False)])
def test_linear_decode_gemv(q, M, dq):
    """M <= 16 runs the decode GEMV kernel for the forward product."""
    _layer(q, M, 4096, 4096, 16, dq, 3300 + M, check_dx=False)


@pytest.mark.parametrize("N,K,r,dq", [(256, 256, 8, True), (130, 192, 64, False)])
def test_merge_and_requantize(q, N, K, r, dq):
    import torch
    W = workloads.custom(3400 + N + K, (N, K), 0.02)
    A = workloads.custom(3401 + N + K, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(3402 + N + K, (r, N), 0.01)
    alpha = 2.0 * r
    say(f"[fp4 merge] N={N} K={K} r={r} double_quant={dq}")
    w = q.quantize(dev_bf16(W), double_quant=dq, quant_type="fp4")
    out = q.merge(w, dev_bf16(A), dev_bf16(B), alpha)
    w2 = q.quantize(out, double_quant=dq, quant_type="fp4")
    torch.cuda.synchronize()
    if dq:
        p, q8, a2 = fp4.quantize(W)
        Wh = fp4.dequantize(p, q8, a2, N, K)
    else:
        p, a = fp4.quantize_nodq(W)
        Wh = fp4.dequantize_nodq(p, a, N, K)
    ref = merge.merge(Wh, A, B, alpha, r)
    got = host_bits(out)
    assert np.array_equal(got, ref), f"merged weight differs at {np.flatnonzero(got != ref)[:8]}"
    rc = fp4.quantize(ref)[0] if dq else fp4.quantize_nodq(ref)[0]
    assert np.array_equal(w2.codes.cpu().numpy(), rc)
