"""The library's calls under HIP graph capture.

Nothing in the library allocates or clears memory with a memset: every call is
plain kernel launches on the caller's stream, writing the caller's buffers and
workspace.  A captured quantize + forward + backward of one layer must
therefore replay to exactly the results of the same calls made eagerly, replay
after replay, with other eager work and synchronisations in between (every
kernel is deterministic: the split sums are added in a fixed order).
"""
import numpy as np
import pytest

from bit_nf4_quantized_15_amd import workloads

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_15_amd import qlora
    return qlora


@pytest.mark.parametrize("M", [64, 8])          # tiled GEMMs, decode GEMV for the forward
def test_captured_layer_replays_match_eager(q, M):
    import torch
    N, K, r, alpha = 320, 512, 16, 32.0
    dev = "cuda:0"
    W = dev_bf16(workloads.custom(7000 + M, (N, K), 0.02))
    x = dev_bf16(workloads.custom(7001 + M, (M, K), 1.0))
    A = dev_bf16(workloads.custom(7002 + M, (K, r), 0.25))
    B = dev_bf16(workloads.custom(7003 + M, (r, N), 0.01))
    dy = dev_bf16(workloads.custom(7004 + M, (M, N), 1.0))
    w = q.NF4Weight.empty(N, K, dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((K, r), dtype=torch.float32, device=dev)
    dB = torch.empty((r, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(q.fwd_workspace(M, N, K, r), q.bwd_workspace(M, N, K, r)), dtype=torch.uint8, device=dev)

    def layer():
        q.quantize(W, out=w)
        q.linear_fwd(w, x, A, B, alpha, y=y, t=t, ws=ws)
        q.linear_bwd(w, x, A, B, alpha, dy, t=t, dx=dx, dA=dA, dB=dB, ws=ws)

    def snapshot():
        torch.cuda.synchronize()
        return [v.detach().clone().cpu() for v in (w.codes, w.q8, w.a2, y, t, dx, dA, dB)]

    say(f"[graph] eager M={M}")
    layer()
    eager = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()                                     # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(3):
        for v in (y, t, dx, dA, dB):               # eager work between replays: clobber every output
            v.fill_(float("nan"))
        w.codes.zero_(); w.q8.zero_(); w.a2.zero_()
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}")
        g.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), f"replay {rep}: output {i} differs"


def test_captured_grouped_schedule_replays_match_eager(q):
    """The training step's grouped schedule (t of a group in one launch, the forward GEMMs, u of the group
    in one launch, the dx GEMMs, every layer's dA and dB in one launch) replays bit for bit."""
    import torch
    M, r, alpha = 200, 24, 48.0
    shapes = [(320, 512), (192, 512), (512, 256)]          # (N, K); the first two share x
    dev = "cuda:0"
    L = []
    for i, (N, K) in enumerate(shapes):
        d = dict(N=N, K=K)
        d["W"] = dev_bf16(workloads.custom(7100 + i, (N, K), 0.02))
        d["x"] = dev_bf16(workloads.custom(7110 + (0 if i < 2 else i), (M, K), 1.0))
        d["A"] = dev_bf16(workloads.custom(7120 + i, (K, r), 0.25))
        d["B"] = dev_bf16(workloads.custom(7130 + i, (r, N), 0.01))
        d["dy"] = dev_bf16(workloads.custom(7140 + i, (M, N), 1.0))
        d["w"] = q.quantize(d["W"])
        for k, shp, dt in (("y", (M, N), torch.bfloat16), ("t", (M, r), torch.bfloat16), ("u", (M, r), torch.bfloat16),
                           ("dx", (M, K), torch.bfloat16), ("dA", (K, r), torch.float32), ("dB", (r, N), torch.float32)):
            d[k] = torch.empty(shp, dtype=dt, device=dev)
        L.append(d)
    groups = [[0, 1], [2]]
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=dev)
    gws = torch.empty(1 << 22, dtype=torch.uint8, device=dev)

    def step():
        for g in groups:
            q.lora_down_batch([(L[i]["x"], L[i]["A"]) for i in g], alpha, t=[L[i]["t"] for i in g], ws=ws)
            for i in g:
                q.fused_gemm_fwd(L[i]["w"], L[i]["x"], L[i]["t"], L[i]["B"], y=L[i]["y"])
        for g in groups:
            q.lora_u_batch([(L[i]["dy"], L[i]["B"]) for i in g], alpha, u=[L[i]["u"] for i in g], ws=ws)
            for i in g:
                q.fused_gemm_bwd_dx(L[i]["w"], L[i]["dy"], L[i]["u"], L[i]["A"], dx=L[i]["dx"])
        q.lora_grads_batch([(d["x"], d["t"], d["u"], d["dy"]) for d in L], dA=[d["dA"] for d in L],
                           dB=[d["dB"] for d in L], ws=gws)

    outs = [d[k] for d in L for k in ("y", "t", "u", "dx", "dA", "dB")]

    def snapshot():
        torch.cuda.synchronize()
        return [v.detach().clone().cpu() for v in outs]

    say("[graph] grouped schedule, eager")
    step()
    eager = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for v in outs:
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[graph] grouped schedule, replay {rep}")
        g.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"
