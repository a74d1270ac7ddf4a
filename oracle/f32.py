"""IEEE binary32 (fp32) as raw uint32 bit patterns: the third compute dtype.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"bitsandbytes deep dive" 8.3 lists fp32 beside bf16 and fp16 as a compute
dtype of a 4-bit layer.  With fp32 every floating-point tensor of the layer
(source weight, dequantized weight, activations, LoRA factors, outputs and
gradients) is binary32.  Nothing is rounded to a 16-bit format: the
dequantized weight is the fp32 product fl32(a_hat * c_q) itself.  The same
three functions as the bf16 and fp16 codecs are offered so that the quantizer
can take any of the three; the fp32 "rounding" is the identity.
"""
import numpy as np

BITS = np.uint32


def to_f32(u32):
    """Exact value of fp32 bit patterns as float32."""
    return np.asarray(u32, dtype=np.uint32).view(np.float32)


def to_f64(u32):
    """Exact value of fp32 bit patterns as float64."""
    return to_f32(u32).astype(np.float64)


def from_f32_rne(f32):
    """fp32 values as their own bit patterns (no rounding: the format is binary32 itself)."""
    return np.ascontiguousarray(np.asarray(f32, dtype=np.float32)).view(np.uint32)


def from_f64(x):
    """Round float64 values to fp32 (nearest, ties to even) and return the bits; for building inputs."""
    return from_f32_rne(np.asarray(x, dtype=np.float64).astype(np.float32))
