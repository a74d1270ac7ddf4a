"""Parity of qlora_quantize / qlora_dequantize (HIP) with the CPU oracle.

Bar: packed codes, q8, a2 and the dequantized bf16 weight bit-exact.
Every case compares the whole weight: the small and ragged shapes, and the
full-size weights of every workload, including the three 235M-weight layers of
the 70B-like MLP (about 20 s of oracle time each).  Output buffers start out
poisoned (tests/conftest.py), so a byte the kernel never writes cannot pass.
"""
import numpy as np
import pytest

from oracle import bf16, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _gpu_quant(q, W):
    w = q.quantize(dev_bf16(W))
    wh = q.dequantize(w)
    import torch
    torch.cuda.synchronize()
    return (w.codes.cpu().numpy(), w.q8.cpu().numpy(), w.a2.cpu().numpy(), host_bits(wh))


def _check_full(q, W, tag):
    N, K = W.shape
    say(f"[quantize] {tag} N={N} K={K}")
    codes, q8, a2, wh = _gpu_quant(q, W)
    rc, rq, ra = nf4.quantize(W)
    assert np.array_equal(codes, rc), f"{tag}: codes differ at {np.flatnonzero(codes != rc)[:8]}"
    assert np.array_equal(q8, rq), f"{tag}: q8 differ at {np.flatnonzero(q8 != rq)[:8]}"
    assert np.array_equal(a2.view(np.uint32), ra.view(np.uint32)), f"{tag}: a2 differ"
    rwh = nf4.dequantize(rc, rq, ra, N, K)
    assert np.array_equal(wh, rwh), f"{tag}: dequant differs at {np.flatnonzero(wh != rwh)[:8]}"


def test_c1_linear_256(q):
    _check_full(q, workloads.weight(workloads.LINEAR_256), workloads.LINEAR_256)


def test_c2_q_proj_with_outliers(q):
    _check_full(q, workloads.weight(workloads.Q_PROJ_DECODE), workloads.Q_PROJ_DECODE)


@pytest.mark.parametrize("N,K", [(1, 64), (3, 192), (5, 640), (257, 64), (64, 11008), (7, 16384 + 64)])
def test_ragged_shapes(q, N, K):
    """Block counts that are not a multiple of 256 (short last group, groups straddling rows)."""
    _check_full(q, workloads.custom(100 + N + K, (N, K), 0.02), f"ragged {N}x{K}")


def test_edge_blocks(q):
    """All-zero block and group, +-0, absmax with both signs, values on levels, subnormal
    and huge scales, planted q8 ties (a2 = 510, a odd), a block whose q8 is 0."""
    rng = np.random.default_rng(1234)
    K = 64 * 8
    # row 0: assorted blocks
    r0 = rng.standard_normal(K).astype(np.float32) * 0.02
    r0[0:64] = 0.0                                          # all-zero block
    r0[64:128] = -0.0
    r0[64 + 3] = 0.0
    r0[128 + 5], r0[128 + 9] = 0.5, -0.5                   # absmax with both signs
    lv = np.array([float(v) for v in nf4.nf4_table()], np.float32)
    r0[192:208] = lv * 4.0                                  # exactly on the levels, a = 4
    r0[256:320] = (rng.standard_normal(64) * 1e-39).astype(np.float32)   # subnormal weights
    r0[320:384] = (rng.standard_normal(64) * 1e36).astype(np.float32)
    r0[384:448] = 1e-30                                     # q8 = 0 against the 1e36 group max
    # row 1: q8 ties: one block with a = 510, blocks with odd a <= 255
    r1 = np.zeros(K, np.float32)
    r1[0] = 510.0
    for j, a in enumerate([1.0, 3.0, 5.0, 101.0, 255.0, 127.0, 63.0]):
        r1[64 * (j + 1)] = a
        r1[64 * (j + 1) + 1] = -a / 3
    # group layout (K = 512: 8 blocks per row, 32 rows per group of 256 blocks):
    # group 0 = row 0 + filler, group 1 = the q8-tie row + zeros (max 510),
    # group 2 = all zero, then a short last group of filler
    filler = bf16.to_f32(workloads.custom(55, (36, K), 0.02))
    W = np.concatenate([r0[None, :], filler[:31], r1[None, :], np.zeros((31, K), np.float32),
                        np.zeros((32, K), np.float32), filler[31:]], axis=0)
    W = bf16.from_f32_rne(W)
    _check_full(q, W, "edge blocks")


@pytest.mark.parametrize("cfg", [workloads.UP_PROJ_M2048, workloads.BLOCK_7B])
def test_full_size_workloads(q, cfg):
    for li, (name, N, K) in enumerate(workloads.CONFIGS[cfg]["layers"]):
        _check_full(q, workloads.weight(cfg, li), f"{cfg} {name}")


@pytest.mark.slow
@pytest.mark.parametrize("layer", [0, 1, 2])
def test_c5_full_layers(q, layer):
    """70B-like MLP weights (235M weights each, deep dive 5.2 and 7.2): codes, q8, a2 and the dequantized
    weight of the whole layer bit-exact against the oracle's full quantization of the same weight."""
    name, N, K = workloads.CONFIGS[workloads.MLP_70B]["layers"][layer]
    _check_full(q, workloads.weight(workloads.MLP_70B, layer), f"{workloads.MLP_70B} {name}")


@pytest.mark.parametrize("cb,dq", [("nf4", True), ("nf4", False), ("fp4", True), ("fp4", False)])
def test_dequantize_fp32_products(q, cb, dq):
    """qlora_dequantize_f32: the fp32 products fl32(a_hat * c_q) bit for bit, on ragged groups."""
    import torch
    from oracle import fp4
    N, K = 37, 640                                          # 370 blocks: one full group and a short one
    W = workloads.custom(6100 + dq, (N, K), 0.02)
    say(f"[dequantize fp32] {cb} double_quant={dq}")
    w = q.quantize(dev_bf16(W), double_quant=dq, quant_type=cb)
    got = q.dequantize(w, fp32=True)
    torch.cuda.synchronize()
    table = nf4.nf4_table() if cb == "nf4" else fp4.fp4_table()
    mod = nf4 if cb == "nf4" else fp4
    if dq:
        p, q8, a2 = mod.quantize(W)
        ref = nf4.dequantize_f32(p, q8, a2, N, K, table=table)
    else:
        p, a = mod.quantize_nodq(W)
        ref = nf4.dequantize_nodq_f32(p, a, N, K, table=table)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), \
        f"differs at {np.flatnonzero(g.view(np.uint32) != ref.view(np.uint32))[:8]}"


def test_batch_matches_per_weight_quantize_and_the_oracle(q):
    """qlora_quantize_batch: 19 weights in one call (runs of one configuration, a run split at 16
    weights, ragged groups, NF4 and FP4, with and without double quantization, bf16 and fp16) give
    the states of one qlora_quantize per weight, byte for byte; the first two also equal the
    oracle's."""
    import torch
    shapes = [(3, 192), (257, 64), (64, 1088), (5, 640)] * 4 + [(7, 16384 + 64), (1, 64), (96, 256)]
    cfgs = [("nf4", True, torch.bfloat16)] * 17 + [("fp4", False, torch.bfloat16), ("nf4", True, torch.float16)]
    Ws, ref, outs = [], [], []
    for i, ((N, K), (cb, dq, dt)) in enumerate(zip(shapes, cfgs)):
        W = dev_bf16(workloads.custom(900 + i, (N, K), 0.02)).to(dt)
        Ws.append(W)
        ref.append(q.quantize(W, double_quant=dq, quant_type=cb))
        outs.append(q.NF4Weight.empty(N, K, W.device, dq, cb, dt))
    say(f"[quantize batch] {len(Ws)} weights")
    q.quantize_batch(Ws, outs)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, outs)):
        assert torch.equal(a.codes, b.codes), f"weight {i}: codes differ"
        assert torch.equal(a.a2.view(torch.int32), b.a2.view(torch.int32)), f"weight {i}: a2 differ"
        assert (a.q8 is None) == (b.q8 is None) and (a.q8 is None or torch.equal(a.q8, b.q8)), f"weight {i}: q8"
    for i in range(2):
        rc, rq, ra = nf4.quantize(workloads.custom(900 + i, shapes[i], 0.02))
        assert np.array_equal(outs[i].codes.cpu().numpy(), rc) and np.array_equal(outs[i].q8.cpu().numpy(), rq)
        assert np.array_equal(outs[i].a2.cpu().numpy().view(np.uint32), ra.view(np.uint32))
