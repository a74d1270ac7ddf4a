"""CPU oracle for the NF4 frozen-base linear layer with a LoRA side branch.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU path computes.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  It shares no code, table, constant generator or helper with the HIP
library in ``bit_nf4_quantized_15_amd``, and it imports nothing from that
package: inputs (seeded synthetic tensors) are handed in by the caller.

Sources (web pages on QLoRA / NF4 / bitsandbytes):

* "bitsandbytes deep dive" (aicoding.csdn.net), section 5.2 "how a 4-bit block
  is encoded": per-block absmax a = max|w|, u = w/a, q = argmin_j |u - c_j|,
  w_hat = a * c_q; block size 64 (section 5.1); two codes per uint8.
* same page, section 6.2: the NF4 codebook is built from quantiles of N(0,1),
  normalised to [-1, 1], asymmetric, with an exact zero.
* same page, section 7.2: double quantization -- 8-bit first-level scales, one
  fp32 second-level scale per 256 first-level scales;
  8/64 + 32/(64*256) = 0.127 bit per parameter (section 7.1, 9.5: without it,
  one fp32 scale per block, 0.5 bit per parameter).
* same page, section 12.2 / 12.4 and "LoRA, QLoRA, QA-LoRA explained"
  (ludovicoyin.github.io), section 2: y = x dequant(W4) + (alpha/r) x A B,
  A: [Din, r], B: [r, Dout]; the base is frozen (no dW).

Modules:
  bf16   -- bf16 decode and round-to-nearest-even encode (own implementation)
  f16    -- fp16 decode and encode (numpy's IEEE binary16), the other 16-bit compute dtype
  f32    -- fp32 bit patterns, the third compute dtype (no rounding of the dequantized weight)
  nf4    -- codebook, blocking, codes, packing, double quantization, dequant
  brute  -- exact rational (fractions.Fraction) brute-force versions
  lora   -- fp64 forward / backward of the QLoRA linear
  merge  -- the LoRA merge W_eff = W_hat + (alpha/r) (A B)^T for deployment
  fp4    -- the fp4 quant type: E2M1 4-bit float levels / 6 in the same scheme
"""
