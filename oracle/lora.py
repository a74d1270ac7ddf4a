"""Forward and backward of the QLoRA linear in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Shapes (LoRA convention of "LoRA, QLoRA, QA-LoRA explained", section 1, and
"bitsandbytes deep dive", section 12.2): x [M, K=Din], W_hat as the [K, N=Dout]
view of the stored [N, K] dequantized weight, A [K, r], B [r, N], s = alpha/r.

Forward (deep dive 12.4; explained, section 2: W_eff = dequant(W4) + (alpha/r) A B):
    y = x W_hat + s (x A) B
Backward: the base weight is frozen (requires_grad = False, deep dive 12.4), so
there is no dW; by the chain rule through the same graph
    u  = s dy B^T                (gradient reaching the LoRA bottleneck)
    dx = dy W_hat^T + u A^T
    dA = x^T u      = s x^T (dy B^T)
    dB = t^T dy     with t = s x A
No bias, no dropout (no workload asks for them).  Every product is a float64
numpy matmul of the exact bf16 input values.

The QA-LoRA pooled branch (same page, sections 3-5) replaces x A by pool(x) A,
pool averaging each group of g consecutive input columns, A [K/g, r]:
    y = x W_hat + s pool(x) A B
"""
import numpy as np


def lora_scale(alpha, r):
    """s = alpha / r (deep dive 12.2: s follows lora_alpha / r)."""
    return float(alpha) / float(r)


def lora_branch(x, A, B, s):
    """s (x A) B -- the low-rank side path."""
    return s * ((np.asarray(x, np.float64) @ np.asarray(A, np.float64)) @ np.asarray(B, np.float64))


def linear_fwd(x, W_hat_nk, A, B, alpha, r):
    """y = x W_hat + s (x A) B; W_hat_nk is the stored [N, K] dequantized weight (float64).

    Returns (y [M, N], t = s x A [M, r]).
    """
    x = np.asarray(x, np.float64)
    s = lora_scale(alpha, r)
    t = s * (x @ np.asarray(A, np.float64))
    y = x @ np.asarray(W_hat_nk, np.float64).T + t @ np.asarray(B, np.float64)
    return y, t


def linear_bwd(x, W_hat_nk, A, B, alpha, r, dy):
    """Gradients of <dy, y> w.r.t. x, A and B (no dW: the base is frozen).

    Returns (dx [M, K], dA [K, r], dB [r, N]).
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    s = lora_scale(alpha, r)
    u = s * (dy @ B.T)
    dx = dy @ np.asarray(W_hat_nk, np.float64) + u @ A.T
    dA = x.T @ u
    dB = (s * (x @ A)).T @ dy
    return dx, dA, dB


def lora_grads(x, A, B, alpha, r, dy):
    """dA, dB alone (the dx-free part of linear_bwd), for sampled full-size checks.

    Same formulas: u = s dy B^T, dA = x^T u, dB = (s x A)^T dy.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    s = lora_scale(alpha, r)
    return x.T @ (s * (dy @ B.T)), (s * (x @ A)).T @ dy


def rel_err(got, ref):
    """Normwise relative error ||got - ref||_F / ||ref||_F (0 when both are zero)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ----------------------------------------------------------------------------
# QA-LoRA pooled branch ("LoRA, QLoRA, QA-LoRA explained", sections 3-5)
# ----------------------------------------------------------------------------
def pool(x, g):
    """pool(x): the mean of each group of g consecutive input columns, [M, K] -> [M, K/g] (section 3)."""
    x = np.asarray(x, np.float64)
    M, K = x.shape
    assert K % g == 0
    return x.reshape(M, K // g, g).mean(axis=2)


def pooled_fwd(x, W_hat_nk, A, B, alpha, r, g):
    """y = x W_hat + s pool(x) A B with A [K/g, r] (section 3: y = x W + pool(x) A B; s = alpha/r as in
    the plain branch).  Returns (y [M, N], t = s pool(x) A [M, r])."""
    x = np.asarray(x, np.float64)
    s = lora_scale(alpha, r)
    t = s * (pool(x, g) @ np.asarray(A, np.float64))
    y = x @ np.asarray(W_hat_nk, np.float64).T + t @ np.asarray(B, np.float64)
    return y, t


def pooled_bwd(x, W_hat_nk, A, B, alpha, r, g, dy):
    """Gradients of <dy, y> for the pooled branch (chain rule through pool, which is linear):
        u  = s dy B^T
        dx = dy W_hat^T + unpool(u A^T) / g    (each group's g columns get the group's value / g)
        dA = pool(x)^T u,   dB = t^T dy
    Returns (dx [M, K], dA [K/g, r], dB [r, N])."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    s = lora_scale(alpha, r)
    u = s * (dy @ B.T)
    dx = dy @ np.asarray(W_hat_nk, np.float64) + np.repeat(u @ A.T, g, axis=1) / g
    px = pool(x, g)
    dA = px.T @ u
    dB = (s * (px @ A)).T @ dy
    return dx, dA, dB
