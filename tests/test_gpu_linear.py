"""Parity of qlora_linear_fwd / qlora_linear_bwd (HIP) with the fp64 CPU oracle.

Bar (normwise relative error, bf16 inputs, fp32 accumulation): y, t, dx, dA,
dB <= 5e-3.  The oracle quantizes W itself (no GPU-produced codes are used as
oracle input).  Small and ragged shapes are checked in full; the full-size
workloads on sampled rows/columns of y and dx (computed one by one by the
oracle) and in full for dA and dB; there the full y, t and dx are also checked to
be finite everywhere, and the whole quantized state bit-exact.  Every output
buffer starts out as NaN (tests/conftest.py), so an element that no kernel
writes fails.
"""
import numpy as np
import pytest

from oracle import bf16, lora, nf4
from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, host_bits, host_f64, say

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _run_gpu(q, W, x, A, B, dy, alpha, want_dx=True, pass_t=True):
    import torch
    w = q.quantize(dev_bf16(W))
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    dx, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t if pass_t else None, need_dx=want_dx)
    torch.cuda.synchronize()
    out = dict(y=host_f64(y), t=host_f64(t), dA=host_f64(dA), dB=host_f64(dB))
    if want_dx:
        out["dx"] = host_f64(dx)
    return out


def _check_full(q, W, x, A, B, dy, alpha, tag, pass_t=True):
    N, K = W.shape
    M, r = x.shape[0], A.shape[1]
    say(f"[linear] {tag} M={M} N={N} K={K} r={r}")
    g = _run_gpu(q, W, x, A, B, dy, alpha, pass_t=pass_t)
    p, q8, a2 = nf4.quantize(W)
    Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
    xf, Af, Bf, dyf = (bf16.to_f64(v) for v in (x, A, B, dy))
    y, t = lora.linear_fwd(xf, Wh, Af, Bf, alpha, r)
    dx, dA, dB = lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
    errs = {k: lora.rel_err(g[k], ref) for k, ref in (("y", y), ("t", t), ("dx", dx), ("dA", dA), ("dB", dB))}
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{tag}: {k} rel err {e:.3e}"
    return errs


def test_c1_single_linear(q):
    c = workloads.LINEAR_256
    _check_full(q, workloads.weight(c), workloads.activations(c), workloads.lora_A(c), workloads.lora_B(c),
                workloads.grad_output(c), workloads.CONFIGS[c]["alpha"], c)


@pytest.mark.parametrize("M,N,K,r", [
    (1, 64, 64, 8), (2, 200, 192, 16), (15, 320, 320, 13), (16, 256, 512, 64),
    (17, 130, 128, 8), (300, 520, 384, 64), (257, 256, 256, 100), (64, 72, 11008 // 4, 32),
])
def test_ragged_shapes(q, M, N, K, r):
    seed = 10 * M + N + K + r
    W = workloads.custom(seed, (N, K), 0.02)
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    _check_full(q, W, x, A, B, dy, 2.0 * r, f"ragged {M}x{N}x{K} r{r}")


@pytest.mark.parametrize("M,N,K,r", [(64, 72, 64 * 43, 16), (9, 260, 320, 8)])
def test_groups_straddling_a_block_pair(q, M, N, K, r):
    """Odd blocks per row: a pair of adjacent blocks of one row can fall into two
    groups of 256 first-level scales (deep dive 7.2), each with its own
    second-level scale.  Weights in every other group are 100x larger, so a block
    dequantized with its neighbour group's scale is off by 100x."""
    seed = 7 * M + N + K
    W = workloads.custom(seed, (N, K), 0.02)
    KB = K // 64
    flat = np.arange(N)[:, None] * KB + np.arange(KB)[None, :]          # flat block index
    big = np.repeat((flat >> 8) & 1, 64, axis=1).astype(bool)
    Wf = bf16.to_f64(W)
    Wf[big] *= 100.0
    W = bf16.from_f32_rne(Wf.astype(np.float32))
    x = workloads.custom(seed + 1, (M, K), 1.0)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    _check_full(q, W, x, A, B, dy, 2.0 * r, f"straddle {M}x{N}x{K} r{r}")


@pytest.mark.parametrize("M,N,K,r", [(17, 130, 128, 8), (300, 520, 384, 64), (64, 72, 64 * 43, 16), (256, 256, 512, 100)])
def test_fused_gemm_bwd_dx_alone(q, M, N, K, r):
    """qlora_fused_gemm_bwd_dx for a given bf16 u: dx = dy W_hat^T + u A^T.  u is the oracle's
    s dy B^T rounded to bf16, the reference uses that same u."""
    import torch
    seed = 20 * M + N + K + r
    W = workloads.custom(seed, (N, K), 0.02)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[bwd dx alone] M={M} N={N} K={K} r={r}")
    dyf, Af, Bf = bf16.to_f64(dy), bf16.to_f64(A), bf16.to_f64(B)
    u = bf16.from_f32_rne(((alpha / r) * (dyf @ Bf.T)).astype(np.float32))
    w = q.quantize(dev_bf16(W))
    dx = q.fused_gemm_bwd_dx(w, dev_bf16(dy), dev_bf16(u), dev_bf16(A))
    torch.cuda.synchronize()
    p, q8, a2 = nf4.quantize(W)
    Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
    ref = dyf @ Wh + bf16.to_f64(u) @ Af.T
    e = lora.rel_err(host_f64(dx), ref)
    say(f"    rel error dx {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("M,N,K,r", [(17, 72, 128, 8), (300, 200, 384, 16), (300, 192, 256, 16)])
def test_bwd_dx_reads_nothing_past_dy(q, M, N, K, r):
    """dy is the head of a larger buffer whose tail is NaN: the dx stage must read nothing past
    dy's own M x N elements (partial column steps when N % 64 != 0, the last row panel when M % 256
    != 0), or the NaN would reach dx through the zero weights of the padding."""
    import torch
    seed = 30 * M + N + K + r
    W = workloads.custom(seed, (N, K), 0.02)
    A = workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r)))
    B = workloads.custom(seed + 3, (r, N), 0.01)
    dy = workloads.custom(seed + 4, (M, N), 1.0)
    alpha = 2.0 * r
    say(f"[bwd dx, NaN past dy] M={M} N={N} K={K} r={r}")
    dyf, Af, Bf = bf16.to_f64(dy), bf16.to_f64(A), bf16.to_f64(B)
    u = bf16.from_f32_rne(((alpha / r) * (dyf @ Bf.T)).astype(np.float32))
    big = torch.full((M * N + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    big[: M * N].copy_(dev_bf16(dy).reshape(-1))
    dyv = big[: M * N].view(M, N)
    w = q.quantize(dev_bf16(W))
    dx = q.fused_gemm_bwd_dx(w, dyv, dev_bf16(u), dev_bf16(A))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dx).all()), "NaN past the end of dy reached dx"
    p, q8, a2 = nf4.quantize(W)
    Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
    e = lora.rel_err(host_f64(dx), dyf @ Wh + bf16.to_f64(u) @ Af.T)
    say(f"    rel error dx {e:.3e}")
    assert e <= TOL


def test_recomputed_t_and_no_dx(q):
    M, N, K, r = 40, 192, 256, 16
    W = workloads.custom(1, (N, K), 0.02); x = workloads.custom(2, (M, K), 1.0)
    A = workloads.custom(3, (K, r), 0.25); B = workloads.custom(4, (r, N), 0.01)
    dy = workloads.custom(5, (M, N), 1.0)
    _check_full(q, W, x, A, B, dy, 32.0, "t recomputed", pass_t=False)
    g = _run_gpu(q, W, x, A, B, dy, 32.0, want_dx=False)
    assert "dx" not in g


def test_lora_off_matches_dequant_product(q):
    """B = 0: y must equal x W_hat on the GPU as well (same tolerance)."""
    M, N, K, r = 64, 256, 256, 8
    W = workloads.custom(11, (N, K), 0.02); x = workloads.custom(12, (M, K), 1.0)
    A = workloads.custom(13, (K, r), 0.3); B = np.zeros((r, N), np.uint16)
    dy = workloads.custom(14, (M, N), 1.0)
    _check_full(q, W, x, A, B, dy, 16.0, "B=0")


def test_c2_decode(q):
    c = workloads.Q_PROJ_DECODE
    W = workloads.weight(c)
    for M in (1, 16):
        _check_full(q, W, workloads.activations(c, M=M), workloads.lora_A(c), workloads.lora_B(c),
                    workloads.grad_output(c, M=M), workloads.CONFIGS[c]["alpha"], f"{c} M={M}")


# ---------------------------------------------------------------- full-size, sampled
def _block_cols(packed, q8, a2, N, K, kb):
    """Oracle dequant of the whole column band of blocks kb (list) over all rows: [N, 64*len(kb)]."""
    bpr = K // nf4.BLOCK
    bidx = (np.arange(N)[:, None] * bpr + np.asarray(kb)[None, :]).reshape(-1)
    ahat = nf4._ahat_of_blocks(q8, a2, bidx)
    pk = packed.reshape(-1, nf4.BLOCK // 2)[bidx].reshape(-1)
    return bf16.to_f64(nf4.dequant_blocks(pk, ahat)).reshape(N, -1)


def _check_sampled(q, cfg, layer, seed=0):
    import torch
    name, N, K = workloads.CONFIGS[cfg]["layers"][layer]
    C = workloads.CONFIGS[cfg]
    M, r, alpha = C["M"], C["r"], C["alpha"]
    say(f"[linear] {cfg} {name} M={M} N={N} K={K} r={r} (sampled)")
    W = workloads.weight(cfg, layer)
    x = workloads.activations(cfg, layer); A = workloads.lora_A(cfg, layer)
    B = workloads.lora_B(cfg, layer); dy = workloads.grad_output(cfg, layer)
    w = q.quantize(dev_bf16(W))
    xd, Ad, Bd, dyd = dev_bf16(x), dev_bf16(A), dev_bf16(B), dev_bf16(dy)
    y, t = q.linear_fwd(w, xd, Ad, Bd, alpha)
    dx, dA, dB = q.linear_bwd(w, xd, Ad, Bd, alpha, dyd, t=t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, 64, replace=False))
    ncols = np.sort(rng.choice(N, 256, replace=False))
    kb = np.sort(rng.choice(K // 64, 4, replace=False))
    kcols = (kb[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    ri = torch.as_tensor(rows, device=y.device)
    g_y = host_f64(y[ri][:, torch.as_tensor(ncols, device=y.device)])
    g_t = host_f64(t[ri])
    g_dx = host_f64(dx[ri][:, torch.as_tensor(kcols, device=y.device)])
    g_dA = host_f64(dA); g_dB = host_f64(dB)
    # every element of the full outputs was written (they start out as NaN) and is finite
    for nm, v in (("y", y), ("t", t), ("dx", dx)):
        assert bool(torch.isfinite(v).all()), f"{cfg} {name}: {nm} holds non-finite (or unwritten) elements"
    g_codes, g_q8, g_a2 = w.codes.cpu().numpy(), w.q8.cpu().numpy(), w.a2.cpu().numpy()
    del w, y, t, dx, dA, dB, xd, dyd
    p, q8, a2 = nf4.quantize(W)
    # the whole quantized state, bit for bit (deep dive 5.2, 7.2)
    assert np.array_equal(g_codes, p) and np.array_equal(g_q8, q8), f"{cfg} {name}: codes / q8 differ"
    assert np.array_equal(g_a2.view(np.uint32), a2.view(np.uint32)), f"{cfg} {name}: a2 differ"
    xf = bf16.to_f64(x[rows]); Af = bf16.to_f64(A); Bf = bf16.to_f64(B); dyf = bf16.to_f64(dy[rows])
    Wn = bf16.to_f64(nf4.dequantize_rows(p, q8, a2, K, ncols))          # W_hat rows for sampled outputs
    y_ref, t_ref = lora.linear_fwd(xf, Wn, Af, Bf[:, ncols], alpha, r)
    Wk = _block_cols(p, q8, a2, N, K, kb)                                # W_hat[:, kcols]
    s = lora.lora_scale(alpha, r)
    dx_ref = dyf @ Wk + (s * (dyf @ Bf.T)) @ Af[kcols].T
    dA_ref, dB_ref = lora.lora_grads(bf16.to_f64(x), Af, Bf, alpha, r, bf16.to_f64(dy))
    errs = dict(y=lora.rel_err(g_y, y_ref), t=lora.rel_err(g_t, t_ref), dx=lora.rel_err(g_dx, dx_ref),
                dA=lora.rel_err(g_dA, dA_ref), dB=lora.rel_err(g_dB, dB_ref))
    say(f"    rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, f"{cfg} {name}: {k} rel err {e:.3e}"


def test_c3_mlp_up_sampled(q):
    _check_sampled(q, workloads.UP_PROJ_M2048, 0)


@pytest.mark.parametrize("layer", [0, 4, 6])
def test_c4_block_layers_sampled(q, layer):
    _check_sampled(q, workloads.BLOCK_7B, layer)


@pytest.mark.slow
@pytest.mark.parametrize("layer", [0, 2])
def test_c5_70b_mlp_sampled(q, layer):
    _check_sampled(q, workloads.MLP_70B, layer)
