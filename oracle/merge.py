"""LoRA merge for deployment: W_eff = W_hat + (alpha/r) (A B)^T in the stored layout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"LoRA, QLoRA, QA-LoRA explained", section 2: the effective weight is
W_eff = dequant(W4) + (alpha/r) A B; the model-compression interview card:
folding the adapter back into the weight removes its inference latency;
"bitsandbytes deep dive", section 12.10: a 4-bit base is merged in higher
precision and may then be re-quantized, which adds error of its own.
Here the stored weight is [N = Dout, K = Din], A is [K, r], B is [r, N], so
    W_eff[n, k] = W_hat[n, k] + s * sum_j A[k, j] B[j, n],   s = alpha / r.
Reading (the pages do not fix the precision): the rank-r sum is accumulated
in fp32 in index order j = 0 .. r-1 (each product of two bf16 values, or of two
fp16 values, is exact in fp32, so each step rounds once), scaled by
s = fl32(alpha/r), added to the dequantized weight in fp32 and rounded once to
the compute dtype (bf16, or fp16 with dtype="f16"; deep dive 8.3).  Re-quantizing is the
ordinary quantize of W_eff (oracle.nf4.quantize / quantize_nodq).
"""
import numpy as np

from . import nf4


def merge(W_hat_u16, A_u16, B_u16, alpha, r, dtype="bf16"):
    """Merged weight [N, K] (uint16 bits of `dtype`) from the dequantized weight W_hat [N, K], A [K, r] and
    B [r, N], all 16-bit bits of `dtype`."""
    c = nf4.codec(dtype)
    Wh = c.to_f32(np.asarray(W_hat_u16, np.uint16))
    A = c.to_f32(np.asarray(A_u16, np.uint16))
    B = c.to_f32(np.asarray(B_u16, np.uint16))
    N, K = Wh.shape
    assert A.shape == (K, r) and B.shape == (r, N)
    acc = np.zeros((N, K), np.float32)
    for j in range(r):
        acc = acc + np.outer(B[j, :], A[:, j]).astype(np.float32)   # exact products, one rounding per step
    s = np.float32(alpha) / np.float32(r)
    w = Wh + (s * acc).astype(np.float32)
    return c.from_f32_rne(w.astype(np.float32))
