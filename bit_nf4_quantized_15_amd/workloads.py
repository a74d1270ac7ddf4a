"""Seeded synthetic workloads: shapes and input tensors, nothing of the method's arithmetic.

This module is the only code shared by the two sides of every parity check
(the HIP library and the CPU oracle both receive the bytes produced here).  It
draws random numbers and rounds them to bf16; it never quantizes, dequantizes
or multiplies anything.

Shapes stand in for the model shapes the QLoRA pages talk about: a 7B-like
d = k = 4096 projection (interview card, LoRA parameter-count example), a
7B-like decoder block with LoRA on every linear layer (deep dive section 12,
target_modules="all-linear"), and 70B-like MLP projections (interview card,
single-GPU 70B fine-tune).  Storage of a weight is [N = Dout, K = Din].

Generation: numpy PCG64 standard normals in float32, drawn in chunks of 2^22
values where chunk c of tensor seed S comes from SeedSequence([S, c]) (so
chunks can be drawn in parallel and a prefix of a tensor does not depend on its
length), scaled by the tensor's standard deviation in float32 and rounded to
bf16 (nearest, ties to even).  Tensor seed = base + 10*layer + id, with the
workload's own base (0, 2000, 3000, 4000, 5000 below) and ids W=0, x=1, A=2,
B=3, dy=4, outlier positions=5.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK = 1 << 22
ID_W, ID_X, ID_A, ID_B, ID_DY, ID_MASK = 0, 1, 2, 3, 4, 5

# The workloads, keyed by what they are: layers [(layer name, N=Dout, K=Din)],
# tokens M, LoRA r, alpha, W std, outlier fraction and factor, seed base
LINEAR_256 = "linear_256x256_m16"
Q_PROJ_DECODE = "q_proj_4096x4096_decode"
UP_PROJ_M2048 = "up_proj_4096x11008_m2048"
BLOCK_7B = "block_7b_7_linears_m4096"
MLP_70B = "mlp_70b_m8192"
CONFIGS = {
    LINEAR_256: dict(workload="single linear 256x256, 16 tokens", layers=[("linear", 256, 256)],
            M=16, r=8, alpha=16.0, w_std=0.02, outlier_frac=0.0, outlier_mult=1.0, base=0),
    Q_PROJ_DECODE: dict(workload="decode GEMV q_proj 4096x4096", layers=[("q_proj", 4096, 4096)],
            M=1, M_alt=16, r=16, alpha=32.0, w_std=0.02, outlier_frac=0.001, outlier_mult=10.0,
            base=2000),
    UP_PROJ_M2048: dict(workload="MLP up-proj 4096->11008, 2048 tokens", layers=[("up_proj", 11008, 4096)],
            M=2048, r=64, alpha=16.0, w_std=0.02, outlier_frac=0.0, outlier_mult=1.0, base=3000),
    BLOCK_7B: dict(workload="7B-like decoder block, 7 linears, 4096 tokens",
            layers=[("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
                    ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                    ("down_proj", 4096, 11008)],
            M=4096, r=64, alpha=16.0, w_std=0.02, outlier_frac=0.0, outlier_mult=1.0, base=4000),
    MLP_70B: dict(workload="70B-like MLP (gate/up 8192->28672, down 28672->8192), 8192 tokens",
            layers=[("gate_proj", 28672, 8192), ("up_proj", 28672, 8192), ("down_proj", 8192, 28672)],
            M=8192, r=64, alpha=16.0, w_std=0.02, outlier_frac=0.0, outlier_mult=1.0, base=5000),
}


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def bf16_bits(f32):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def normal_f32(seed, n):
    """n standard normals (float32) of tensor seed `seed`, chunked as described above."""
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, CHUNK))

    def fill(ci):
        s = starts[ci]
        e = min(n, s + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, ci])))
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)

    if len(starts) <= 1:
        for ci in range(len(starts)):
            fill(ci)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def normal_bf16(seed, shape, std):
    """bf16 (uint16 bits) tensor of N(0, std^2) values."""
    n = int(np.prod(shape))
    v = normal_f32(seed, n)
    if std != 1.0:
        v *= np.float32(std)
    return bf16_bits(v).reshape(shape)


def normal_f16(seed, shape, std):
    """fp16 (uint16 bits) tensor of N(0, std^2) values: the same draws as normal_bf16, rounded to
    binary16 (nearest, ties to even) instead."""
    n = int(np.prod(shape))
    v = normal_f32(seed, n)
    if std != 1.0:
        v *= np.float32(std)
    return v.astype(np.float16).view(np.uint16).reshape(shape)


def normal_fp32(seed, shape, std):
    """fp32 (uint32 bits) tensor of N(0, std^2) values: the same draws as normal_bf16, kept in binary32."""
    n = int(np.prod(shape))
    v = normal_f32(seed, n)
    if std != 1.0:
        v *= np.float32(std)
    return np.ascontiguousarray(v).view(np.uint32).reshape(shape)


def seed_of(wl, layer, tensor_id):
    return CONFIGS[wl]["base"] + 10 * layer + tensor_id


def weight(wl, layer=0):
    """Base weight [N, K] as bf16 bits, with the configured outliers planted."""
    cfg = CONFIGS[wl]
    _, N, K = cfg["layers"][layer]
    n = N * K
    v = normal_f32(seed_of(wl, layer, ID_W), n)
    v *= np.float32(cfg["w_std"])
    if cfg["outlier_frac"] > 0.0:
        count = int(n * cfg["outlier_frac"])
        g = np.random.default_rng(seed_of(wl, layer, ID_MASK))
        pos = g.choice(n, size=count, replace=False)
        v[pos] *= np.float32(cfg["outlier_mult"])
    return bf16_bits(v).reshape(N, K)


def activations(wl, layer=0, M=None):
    """x [M, K] ~ N(0, 1) as bf16 bits."""
    cfg = CONFIGS[wl]
    _, N, K = cfg["layers"][layer]
    M = cfg["M"] if M is None else M
    return normal_bf16(seed_of(wl, layer, ID_X), (M, K), 1.0)


def lora_A(wl, layer=0):
    """A [K, r] ~ N(0, 1/r) as bf16 bits."""
    cfg = CONFIGS[wl]
    _, N, K = cfg["layers"][layer]
    r = cfg["r"]
    return normal_bf16(seed_of(wl, layer, ID_A), (K, r), float(1.0 / np.sqrt(r)))


def lora_B(wl, layer=0):
    """B [r, N] ~ N(0, 0.01^2) as bf16 bits (non-zero on purpose, unlike a fresh init)."""
    cfg = CONFIGS[wl]
    _, N, K = cfg["layers"][layer]
    return normal_bf16(seed_of(wl, layer, ID_B), (cfg["r"], N), 0.01)


def grad_output(wl, layer=0, M=None):
    """dy [M, N] ~ N(0, 1) as bf16 bits."""
    cfg = CONFIGS[wl]
    _, N, K = cfg["layers"][layer]
    M = cfg["M"] if M is None else M
    return normal_bf16(seed_of(wl, layer, ID_DY), (M, N), 1.0)


def custom(seed, shape, std=1.0):
    """Free-form seeded bf16 tensor for edge-case tests (same recipe)."""
    return normal_bf16(seed, shape, std)
