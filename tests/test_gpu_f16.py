"""Parity of the fp16 compute dtype ("bitsandbytes deep dive" 8.3: fp32, bf16 or
fp16) through every entry point, against the CPU oracle with dtype="f16".

Bar: codes, q8, a2 (or the fp32 absmax), the dequantized and the merged fp16
weights bit-exact; y, t, dx, dA, dB within 1e-3 normwise relative error of the
fp64 oracle on the fp16 reconstruction.  The bar follows from the arithmetic:
fp16 inputs and outputs carry a unit roundoff of 2^-11 (4.9e-4) and the sums
accumulate in fp32, so the rounding of y (or t, dx) once contributes about
2^-11 / sqrt(3) normwise; 1e-3 leaves room for t's own rounding feeding y and
stays below what a single stray bf16 rounding (2^-8) anywhere in the path
would cost.  Both codebooks, both scale layouts,
tiled (even and odd block counts) and decode shapes, the QA-LoRA pooled branch
and the stand-alone down-projection.
"""
import numpy as np
import pytest

from oracle import f16, fp4, lora, merge, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_f16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _oracle_quant(W, cb, dq):
    mod = nf4 if cb == "nf4" else fp4
    N, K = W.shape
    if dq:
        p, q8, a2 = mod.quantize(W, dtype="f16")
        return p, q8, a2, mod.dequantize(p, q8, a2, N, K, dtype="f16")
    p, a = mod.quantize_nodq(W, dtype="f16")
    return p, None, a, mod.dequantize_nodq(p, a, N, K, dtype="f16")


@pytest.mark.parametrize("cb", ["nf4", "fp4"])
@pytest.mark.parametrize("N,K,dq", [(256, 256, True), (257, 64, True), (64, 11008, True), (130, 192, False)])
def test_quantize_dequantize(q, cb, N, K, dq):
    import torch
    W = workloads.normal_f16(4100 + N + K, (N, K), 0.02)
    say(f"[f16 quantize] {cb} N={N} K={K} double_quant={dq}")
    w = q.quantize(dev_f16(W), double_quant=dq, quant_type=cb)
    assert w.dtype == torch.float16
    wh = q.dequantize(w)
    torch.cuda.synchronize()
    assert wh.dtype == torch.float16
    p, q8, a2, rwh = _oracle_quant(W, cb, dq)
    assert np.array_equal(w.codes.cpu().numpy(), p)
    if dq:
        assert np.array_equal(w.q8.cpu().numpy(), q8)
    assert np.array_equal(w.a2.cpu().numpy().view(np.uint32), a2.view(np.uint32))
    got = host_bits(wh)
    assert np.array_equal(got, rwh), f"dequant differs at {np.flatnonzero(got != rwh)[:8]}"


def test_edge_blocks(q):
    """All-zero and +-0 blocks, fp16 subnormal weights, weights at the fp16 maximum."""
    import torch
    rng = np.random.default_rng(77)
    K = 64 * 6
    r0 = (rng.standard_normal(K) * 0.02).astype(np.float32)
    r0[0:64] = 0.0
    r0[64:128] = -0.0
    r0[128:192] = (rng.standard_normal(64) * 1e-6).astype(np.float32)      # fp16 subnormals
    r0[192:256] = (rng.standard_normal(64) * 2e4).astype(np.float32)
    r0[192] = 65504.0
    W = np.concatenate([f16.from_f32_rne(r0)[None, :], workloads.normal_f16(78, (40, K), 0.02)], axis=0)
    for cb in ("nf4", "fp4"):
        for dq in (True, False):
            w = q.quantize(dev_f16(W), double_quant=dq, quant_type=cb)
            wh = q.dequantize(w)
            torch.cuda.synchronize()
            p, q8, a2, rwh = _oracle_quant(W, cb, dq)
            assert np.array_equal(w.codes.cpu().numpy(), p), (cb, dq)
            assert np.array_equal(host_bits(wh), rwh), (cb, dq)


def _layer(q, M, N, K, r, cb, dq, seed, check_dx=True):
    import torch
    W = workloads.normal_f16(seed, (N, K), 0.02)
    x = workloads.normal_f16(seed + 1, (M, K), 1.0)
    A = workloads.normal_f16(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.normal_f16(seed + 3, (r, N), 0.01)
    dy = workloads.normal_f16(seed + 4, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[f16 linear] {cb} M={M} N={N} K={K} r={r} double_quant={dq}")
    w = q.quantize(dev_f16(W), double_quant=dq, quant_type=cb)
    xd, Ad, Bd, dyd = dev_f16(x), dev_f16(A), dev_f16(B), dev_f16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    dx, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t, need_dx=check_dx)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16 and t.dtype == torch.float16
    Wh = f16.to_f64(_oracle_quant(W, cb, dq)[3])
    xf, Af, Bf, dyf = (f16.to_f64(v) for v in (x, A, B, dy))
    ry, rt = lora.linear_fwd(xf, Wh, Af, Bf, alpha, r)
    rdx, rdA, rdB = lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
    pairs = [("y", y, ry), ("t", t, rt), ("dA", dA, rdA), ("dB", dB, rdB)]
    if check_dx:
        pairs.append(("dx", dx, rdx))
    errs = {k: lora.rel_err(host_f64(v), ref) for k, v, ref in pairs}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{k} rel err {e:.3e}"
    return w, x, t


@pytest.mark.parametrize("M,N,K,r,cb,dq", [(64, 256, 512, 16, "nf4", True), (300, 520, 384, 64, "nf4", True),
                                           (64, 72, 64 * 43, 16, "fp4", True), (17, 130, 128, 8, "nf4", False),
                                           (257, 256, 256, 100, "fp4", False)])
def test_linear_tiled(q, M, N, K, r, cb, dq):
    _layer(q, M, N, K, r, cb, dq, 4200 + M + N + K + r)


@pytest.mark.parametrize("M,cb,dq", [(1, "nf4", True), (16, "nf4", True), (1, "fp4", False), (5, "fp4", True)])
def test_linear_decode_gemv(q, M, cb, dq):
    _layer(q, M, 4096, 4096, 16, cb, dq, 4300 + M, check_dx=False)


def test_lora_down_standalone_matches_linear_t(q):
    """qlora_lora_down with the fp16 dtype gives the t that qlora_linear_fwd returns."""
    import torch
    w, x, t = _layer(q, 48, 192, 256, 16, "nf4", True, 4400)
    A = workloads.normal_f16(4402, (256, 16), 0.25)
    t2 = q.lora_down(dev_f16(x), dev_f16(A), 32.0)
    torch.cuda.synchronize()
    assert t2.dtype == torch.float16
    assert np.array_equal(host_bits(t2), host_bits(t))


@pytest.mark.parametrize("cb,dq", [("nf4", True), ("fp4", False)])
def test_merge_and_requantize(q, cb, dq):
    import torch
    N, K, r = 256, 192, 16
    W = workloads.normal_f16(4500, (N, K), 0.02)
    A = workloads.normal_f16(4501, (K, r), 0.25)
    B = workloads.normal_f16(4502, (r, N), 0.01)
    alpha = 2.0 * r
    say(f"[f16 merge] {cb} double_quant={dq}")
    w = q.quantize(dev_f16(W), double_quant=dq, quant_type=cb)
    out = q.merge(w, dev_f16(A), dev_f16(B), alpha)
    w2 = q.quantize(out, double_quant=dq, quant_type=cb)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    ref = merge.merge(_oracle_quant(W, cb, dq)[3], A, B, alpha, r, dtype="f16")
    got = host_bits(out)
    assert np.array_equal(got, ref), f"merged weight differs at {np.flatnonzero(got != ref)[:8]}"
    assert np.array_equal(w2.codes.cpu().numpy(), _oracle_quant(ref, cb, dq)[0])


def test_pooled(q):
    import torch
    M, N, K, r, g = 64, 256, 512, 16, 64
    W = workloads.normal_f16(4600, (N, K), 0.02)
    x = workloads.normal_f16(4601, (M, K), 1.0)
    A = workloads.normal_f16(4602, (K // g, r), 0.25)
    B = workloads.normal_f16(4603, (r, N), 0.01)
    dy = workloads.normal_f16(4604, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[f16 pooled] M={M} N={N} K={K} r={r} g={g}")
    w = q.quantize(dev_f16(W))
    xd, Ad, Bd, dyd = dev_f16(x), dev_f16(A), dev_f16(B), dev_f16(dy)
    y, t = q.pooled_fwd(w, xd, Ad, Bd, alpha, g)
    dx, dA, dB = q.pooled_bwd(w, xd, Ad, Bd, alpha, g, dyd, t=t)
    torch.cuda.synchronize()
    Wh = f16.to_f64(_oracle_quant(W, "nf4", True)[3])
    xf, Af, Bf, dyf = (f16.to_f64(v) for v in (x, A, B, dy))
    ry, rt = lora.pooled_fwd(xf, Wh, Af, Bf, alpha, r, g)
    rdx, rdA, rdB = lora.pooled_bwd(xf, Wh, Af, Bf, alpha, r, g, dyf)
    errs = {k: lora.rel_err(host_f64(v), ref) for k, v, ref in
            (("y", y, ry), ("t", t, rt), ("dx", dx, rdx), ("dA", dA, rdA), ("dB", dB, rdB))}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{k} rel err {e:.3e}"


def test_dtype_mismatch_is_rejected(q):
    """A bf16 activation with an fp16 weight state is refused by the binding before any launch."""
    import torch
    W = workloads.normal_f16(4700, (64, 128), 0.02)
    w = q.quantize(dev_f16(W))
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda:0")
    A = torch.zeros((128, 8), dtype=torch.float16, device="cuda:0")
    B = torch.zeros((8, 64), dtype=torch.float16, device="cuda:0")
    with pytest.raises(TypeError):
        q.linear_fwd(w, x, A, B, 16.0)
