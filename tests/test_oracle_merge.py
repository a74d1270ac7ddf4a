"""Pins of the merge oracle (oracle.merge) against the pages and the mathematics.

* the worked rank-1 example of "LoRA, QLoRA, QA-LoRA explained" (section 1,
  a minimal example): with a zero base weight and s = 1 the merged weight is
  Delta W = A B (the effective weight of section 2);
* an exact rational re-derivation (fractions.Fraction) of every rounding step
  on a small case, so the vectorized form cannot transpose an operand, drop the
  scale or round at a different point;
* the merge identity: x W_eff equals the unmerged forward x W_hat + s (x A) B
  up to the rounding of W_eff to bf16.
"""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import bf16, brute, lora, merge, nf4
from bit_nf4_quantized_15_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_rank1_example():
    with open(os.path.join(GOLDEN, "lora_worked_examples.json")) as f:
        ex = json.load(f)["rank1_delta_w"]
    A = bf16.from_f32_rne(np.array(ex["A"], np.float32))            # [Din=4, r=1]
    B = bf16.from_f32_rne(np.array(ex["B"], np.float32))            # [r=1, Dout=2]
    dW = np.array(ex["delta_w"])                                    # [Din, Dout] as printed
    W0 = np.zeros((2, 4), np.uint16)                                # zero base weight, stored [Dout, Din]
    got = bf16.to_f64(merge.merge(W0, A, B, alpha=1.0, r=1))
    # the printed values are decimals; A, B and the result are bf16 (relative rounding <= 2^-8 each)
    assert np.allclose(got, dW.T, rtol=2.0 ** -6, atol=0)


def test_matches_rational_rounding_steps():
    rng = np.random.default_rng(3)
    N, K, r, alpha = 3, 64, 5, 10.0
    W = workloads.custom(41, (N, K), 0.02)
    p, q8, A2 = nf4.quantize(W)
    Wh = nf4.dequantize(p, q8, A2, N, K)
    A = bf16.from_f32_rne((rng.standard_normal((K, r)) / np.sqrt(r)).astype(np.float32))
    B = bf16.from_f32_rne((rng.standard_normal((r, N)) * 0.01).astype(np.float32))
    got = merge.merge(Wh, A, B, alpha, r)
    s = brute.round_f32(Fraction(alpha) / r)
    Af, Bf, Whf = bf16.to_f64(A), bf16.to_f64(B), bf16.to_f64(Wh)
    for n in range(N):
        for k in range(K):
            acc = Fraction(0)
            for j in range(r):
                acc = brute.round_f32(acc + Fraction(float(Af[k, j])) * Fraction(float(Bf[j, n])))
            w = brute.round_f32(Fraction(float(Whf[n, k])) + brute.round_f32(s * acc))
            ref = bf16.from_f32_rne(np.array([float(w)], np.float32))[0]
            assert got[n, k] == ref, (n, k)


def test_merged_forward_identity():
    rng = np.random.default_rng(4)
    M, N, K, r, alpha = 5, 48, 128, 4, 8.0
    W = workloads.custom(42, (N, K), 0.02)
    p, q8, A2 = nf4.quantize(W)
    Wh = nf4.dequantize(p, q8, A2, N, K)
    A = bf16.from_f32_rne((rng.standard_normal((K, r)) / np.sqrt(r)).astype(np.float32))
    B = bf16.from_f32_rne((rng.standard_normal((r, N)) * 0.01).astype(np.float32))
    x = rng.standard_normal((M, K))
    Weff = bf16.to_f64(merge.merge(Wh, A, B, alpha, r))
    y_ref, _ = lora.linear_fwd(x, bf16.to_f64(Wh), bf16.to_f64(A), bf16.to_f64(B), alpha, r)
    assert lora.rel_err(x @ Weff.T, y_ref) < 2.0 ** -8
    # and the correction is really there: without it the error is far larger
    assert lora.rel_err(x @ bf16.to_f64(Wh).T, y_ref) > 16 * lora.rel_err(x @ Weff.T, y_ref)
