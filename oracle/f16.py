"""IEEE binary16 (fp16) as raw uint16 bit patterns.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"bitsandbytes deep dive" 8.3 lists the compute dtypes a 4-bit layer can run
in: fp32, bf16 or fp16.  With fp16 every 16-bit tensor of the layer (the
source weight, the dequantized weight, activations, the LoRA factors and
gradients flowing through it) is binary16: 1 sign bit, 5 exponent bits,
10 stored mantissa bits, with subnormals.  numpy's float16 is that format, and
its conversion from float32 rounds to nearest, ties to even, subnormals
included; it is used here as a library primitive and pinned against torch's
float32 -> float16 cast in the tests.
"""
import numpy as np

BITS = np.uint16     # storage of one value


def to_f32(u16):
    """Exact value of fp16 bit patterns as float32."""
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_f64(u16):
    """Exact value of fp16 bit patterns as float64."""
    return to_f32(u16).astype(np.float64)


def from_f32_rne(f32):
    """Round float32 values to fp16, nearest, ties to even; returns uint16 bits."""
    with np.errstate(over="ignore"):
        return np.asarray(f32, dtype=np.float32).astype(np.float16).view(np.uint16)
