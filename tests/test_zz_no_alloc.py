"""qlora_linear_fwd_noalloc, the forward that allocates nothing (its workspace is the library's fixed
per-GPU array), against qlora_linear_fwd with a workspace of its own: the same kernels on the same
inputs, so y and t must match bit for bit.  Two calls in a row share the array, the second on a
smaller input (a tiled-path call, then a decode-size call), so stale contents from the first call
must not leak into the second.  Output buffers start out poisoned (tests/conftest.py)."""
import numpy as np
import pytest

from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


def _compare(q, seed, M, N, K, r):
    import torch
    W = workloads.custom(seed, (N, K), 0.02)
    x = dev_bf16(workloads.custom(seed + 1, (M, K), 1.0))
    A = dev_bf16(workloads.custom(seed + 2, (K, r), float(1 / np.sqrt(r))))
    B = dev_bf16(workloads.custom(seed + 3, (r, N), 0.01))
    alpha = 2.0 * r
    say(f"[no-alloc] M={M} N={N} K={K} r={r}, workspace {q.fwd_workspace(M, N, K, r)} bytes")
    w = q.quantize(dev_bf16(W))
    y0, t0 = q.linear_fwd(w, x, A, B, alpha)
    y1, t1 = q.linear_fwd_noalloc(w, x, A, B, alpha)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), "y differs"
    assert torch.equal(t0.view(torch.int16), t1.view(torch.int16)), "t differs"
    assert torch.isfinite(y1.float()).all()


def test_noalloc_matches_linear_fwd_on_two_calls(q):
    _compare(q, 9500, 256, 1024, 2048, 16)     # tiled path: split partial sums of t in the array
    _compare(q, 9510, 4, 512, 1024, 8)         # smaller, decode path: published partials and tags


def test_noalloc_rejects_sizes_beyond_the_array(q):
    import torch
    M, N, K, r = 32768, 64, 64, 128
    assert q.fwd_workspace(M, N, K, r) > 4 << 20
    w = q.quantize(dev_bf16(workloads.custom(9520, (N, K), 0.02)))
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    A = torch.zeros((K, r), dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros((r, N), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(q.QLoraError) as e:
        q.linear_fwd_noalloc(w, x, A, B, 1.0)
    assert e.value.status == -4
