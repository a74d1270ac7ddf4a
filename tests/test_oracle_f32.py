"""Pins of the oracle's fp32 compute-dtype path ("bitsandbytes deep dive" 8.3:
fp32, bf16 or fp16) against things other than itself: torch's float32 values,
the rational brute-force encoders (codes and scale codes), exact rational
rounding of the dequantized products, and the bf16 path on weights whose
values are bf16 values.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, f32, fp4, nf4
from bit_nf4_quantized_15_amd import workloads


def test_f32_codec_matches_torch_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]            # finite patterns
    ref = torch.from_numpy(bits.view(np.int32)).view(torch.float32).double().numpy()
    got = f32.to_f64(bits)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(f32.from_f32_rne(f32.to_f32(bits)), bits)


def _f32_blocks(seed, nb):
    """fp32 blocks with values that are not bf16 or fp16 values, subnormals, signed zeros, and weights
    planted on and just above the exact decision thresholds a * m_j (rounded down to fp32)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((nb, 64)) * 0.02).astype(np.float32)
    w[1] = 0.0
    w[2, ::5] = -0.0
    w[3] *= np.float32(1e-37)                                   # fp32 subnormals
    w[4, 9] = 3.0
    w[5] = (rng.standard_normal(64) * 1e30).astype(np.float32)
    for b, mids in ((6, nf4.nf4_midpoints()), (7, fp4.fp4_midpoints())):
        w[b, 0] = 1.7                                           # a = 1.7
        for j, m in enumerate(mids[:31]):
            x = Fraction(float(np.float32(1.7))) * Fraction(float(m))
            v = np.float32(float(x))
            if Fraction(float(v)) > x:
                v = np.nextafter(v, np.float32(-np.inf))      # RD_f32(a m_j)
            w[b, 1 + 2 * j] = v
            w[b, 2 + 2 * j] = np.nextafter(v, np.float32(np.inf))
    return f32.from_f32_rne(w)


@pytest.mark.parametrize("cb", ["nf4", "fp4"])
def test_codes_and_scales_from_f32_weights_match_bruteforce(cb):
    W = _f32_blocks(11, 24)
    wf = f32.to_f64(W)
    mod = nf4 if cb == "nf4" else fp4
    packed, q8, A2 = mod.quantize(W.reshape(4, -1), dtype="f32")
    codes = nf4.unpack_nibbles(packed).reshape(-1, 64)
    for b in range(wf.shape[0]):
        if cb == "nf4":
            assert list(codes[b]) == brute.nf4_codes_block(wf[b], nf4.nf4_table()), b
        else:
            assert list(codes[b]) == brute.fp4_codes_block(wf[b], fp4.fp4_table()), b
    a = np.abs(wf).max(axis=1)
    assert A2.size == 1 and A2[0] == np.float32(a.max())
    for b in range(wf.shape[0]):
        assert q8[b] == brute.scale_code(a[b], A2[0]), b
    packed2, absmax = mod.quantize_nodq(W.reshape(4, -1), dtype="f32")
    assert np.array_equal(packed2, packed)
    assert np.array_equal(absmax, a.astype(np.float32))


def test_bf16_valued_f32_weights_quantize_like_bf16():
    """Codes and scales depend on the values only: an fp32 weight holding bf16 values quantizes exactly as
    the bf16 weight does (a special case that reduces to the pinned bf16 path)."""
    Wb = workloads.custom(62, (16, 512), 0.02)
    vals = nf4.codec("bf16").to_f32(Wb)
    Wf = f32.from_f32_rne(vals)
    for mod in (nf4, fp4):
        pb, qb, Ab = mod.quantize(Wb)
        pf, qf, Af = mod.quantize(Wf, dtype="f32")
        assert np.array_equal(pb, pf) and np.array_equal(qb, qf) and np.array_equal(Ab, Af)


@pytest.mark.parametrize("cb", ["nf4", "fp4"])
def test_f32_dequant_is_the_exactly_rounded_product(cb):
    W = workloads.normal_fp32(63, (8, 256), 0.02)
    mod = nf4 if cb == "nf4" else fp4
    table = nf4.nf4_table() if cb == "nf4" else fp4.fp4_table()
    packed, q8, A2 = mod.quantize(W, dtype="f32")
    got = mod.dequantize(packed, q8, A2, 8, 256, dtype="f32").reshape(-1, 64)
    ah = nf4.scale_dequant(q8, A2)
    codes = nf4.unpack_nibbles(packed).reshape(-1, 64)
    for b in range(codes.shape[0]):
        for i in range(64):
            p = Fraction(float(ah[b])) * Fraction(float(table[codes[b, i]]))
            want = np.float32(float(brute.round_f32(p))) if p != 0 else None
            g = f32.to_f32(got[b, i:i + 1])[0]
            if want is None:
                assert g == 0.0
            else:
                assert g == want, (b, i)


def test_f32_weights_carry_more_than_bf16_precision():
    """fp32 weights are encoded from their own values: rounding them to bf16 first changes some codes
    (the fp32 path does not pass through a 16-bit format)."""
    W = workloads.normal_fp32(64, (64, 1024), 0.02)
    vals = f32.to_f32(W)
    p32, _, _ = nf4.quantize(W, dtype="f32")
    pb, _, _ = nf4.quantize(nf4.codec("bf16").from_f32_rne(vals))
    assert not np.array_equal(p32, pb)
