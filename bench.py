#!/usr/bin/env python3
"""Throughput of the NF4 frozen-base linear + LoRA hot path on one MI355X.

One step = the whole hot path over one batch of the 7B-like decoder block
(q/k/v/o 4096x4096, gate/up 4096->11008, down 11008->4096, LoRA r=64,
alpha=16, M = 4096 tokens): NF4 + double-quant quantization of all seven
weights, the fused forward of all seven layers (LoRA down-projection, fused
dequant GEMM with the LoRA up-projection), and the backward of all seven
(u, dx, dA, dB).  Inputs are seeded synthetic tensors already resident in HBM.

value = algorithmic fwd+bwd FLOP of the seven linears / step time, where a
layer counts 2MKN (forward base) + 2MKN (dx) + 2Mr(K+N) (forward LoRA) +
4Mr(K+N) (backward LoRA); quantization time is inside the step but adds no
FLOP.  Extra fields: the dominant kernel of the step (the fused backward dx
GEMM, timed on its own on the same shapes right after the timed steps)
against the bf16 MFMA roofline, the forward GEMM likewise, quantize /
dequantize bandwidth, the decode forward on q_proj and fused q/k/v and gate/up
weights against HBM bandwidth (the single-launch layer call, the GEMV kernel
alone and a plain read of the same bytes), forward+backward of the up_proj (M=2048) and 70B-like MLP (M=8192)
configs with the quantize rate of the latter's 704.6M weights, the
scale-layout / codebook / dtype variants, a dense bf16 torch.matmul for
context, and the CPU oracle timed on a bounded sample.

usage: python bench.py [--gpus 1] [--steps 10] [--warmup 10] [--no-cpu-baseline]
       python bench.py --mode pmc     (a few untimed steps + a calibration copy, for rocprofv3 --pmc)
       python bench.py --pmc-summary FETCH_CSV WRITE_CSV [--pmc-kernel fwd|bwd_dx]
                                      (HBM bytes per launch of one GEMM kernel from the two
                                       counter runs, scaled by the calibration copy)
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFS = 157.3      # MI355X dense fp32 MFMA
FP32_VECTOR_PEAK_TFS = 157.3   # MI355X fp32 vector (non-matrix) peak
METRIC = "fused NF4-dequant+LoRA linear TFLOP/s (M=4096) and decode GEMV HBM GB/s, 1 MI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip decode / quantize / dense context lines")
    p.add_argument("--mode", choices=["bench", "pmc", "pmc-decode"], default="bench")
    p.add_argument("--schedule", choices=["grouped", "deferred", "per-layer"], default="grouped",
                   help="grouped: the LoRA products t and u of the layers that share their input in one launch "
                        "(qlora_lora_down_batch, qlora_lora_u_batch), the GEMMs per layer, every layer's dA, dB "
                        "in one launch at the end (qlora_lora_grads_batch); deferred: t per layer, u and dx per "
                        "layer (qlora_linear_bwd_dx), dA, dB at the end; per-layer: qlora_linear_fwd's stages and "
                        "qlora_linear_bwd per layer")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    p.add_argument("--pmc-kernel", choices=["fwd", "bwd_dx", "quantize", "gemv", "grads"], default="fwd")
    p.add_argument("--decode-shape", choices=sorted(DECODE_SHAPES), default="gate_up")
    p.add_argument("--decode-m", type=int, default=1)
    p.add_argument("--pmc-counters", metavar="COUNTER_CSV",
                   help="mean per dispatch of every counter in a rocprofv3 --pmc csv, by kernel")
    return p.parse_args()


# consecutive layers of a decoder block that read the same input
SHARED_INPUT = {("q_proj", "k_proj"), ("k_proj", "v_proj"), ("gate_proj", "up_proj")}

HERE = os.path.dirname(os.path.abspath(__file__))
KERNELS = {"fwd": "nf4_gemm_fwd_kernel", "bwd_dx": "nf4_gemm_bwd_dx_kernel", "quantize": "nf4_quantize_batch_kernel",
           "gemv": "nf4_gemv_stream_kernel", "grads": "tnb_kernel"}
_CSRC = os.path.join(HERE, "bit_nf4_quantized_15_amd", "csrc")
SOURCES = {"fwd": "gemm.hip", "bwd_dx": "gemm.hip", "quantize": "quantize.hip", "gemv": "gemv.hip", "grads": "lora.hip"}
WORKLOAD_TAG = {"fwd": "7B_block_7_layers_M4096_r64", "bwd_dx": "7B_block_7_layers_M4096_r64",
                "quantize": "7B_block_7_layers", "gemv": "gate_up_2x11008x4096_M1_r32",
                "grads": "7B_block_7_layers_M4096_r64"}
TRAFFIC_FILES = {k: os.path.join(HERE, "profiles", f"{v}__{WORKLOAD_TAG[k]}__hbm_traffic.txt")
                 for k, v in KERNELS.items()}
CALIB_BYTES = 512 << 20
# the decode shape that the GEMV traffic summary uses: fused gate/up, M = 1
PMC_DECODE = dict(N=22016, K=4096, r=32, M=1)
# decode shapes of --mode pmc-decode (--decode-shape): [layer rows ...], K, r per layer
DECODE_SHAPES = {"q_proj": ([4096], 4096, 16), "qkv": ([4096] * 3, 4096, 16), "gate_up": ([11008] * 2, 4096, 16)}


def gemm_source_sha(kind="fwd"):
    """sha256 of a kernel's source with comments and whitespace removed: a change of
    the code (not of its comments) invalidates the recorded counter figures."""
    import re
    with open(os.path.join(_CSRC, SOURCES[kind])) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def fwd_algorithmic_bytes(layers, M, r):
    """Per-launch HBM bytes the forward GEMM must move, averaged over the layer shapes:
    x, codes, q8, a2, t, B in and y out."""
    tot = 0
    for _, N, K in layers:
        tot += 2 * M * K + N * K // 2 + N * K // 64 + 4 * (-(-N * K // 16384)) + 2 * M * r + 2 * r * N + 2 * M * N
    return tot / len(layers)


def bwd_dx_algorithmic_bytes(layers, M, r):
    """Per-launch HBM bytes the backward dx GEMM must move, averaged over the layer shapes:
    dy, codes, q8, a2, u, A in and dx out."""
    tot = 0
    for _, N, K in layers:
        tot += 2 * M * N + N * K // 2 + N * K // 64 + 4 * (-(-N * K // 16384)) + 2 * M * r + 2 * K * r + 2 * M * K
    return tot / len(layers)


def quantize_algorithmic_bytes(layers):
    """Per-launch HBM bytes of the quantize kernel, which takes every weight of the step in one launch:
    the bf16 weights in, codes, q8 and a2 out."""
    return sum(N * K * 2 + N * K // 2 + N * K // 64 + 4 * (-(-N * K // 16384)) for _, N, K in layers)


def grads_algorithmic_bytes(layers, M, r):
    """HBM bytes of the one gradient launch of a step (every layer's dA and dB): x, dy, u and t in,
    dA and dB (fp32) out."""
    return sum(2 * M * K + 2 * M * N + 2 * 2 * M * r + 4 * K * r + 4 * r * N for _, N, K in layers)


def algorithmic_bytes(kind, layers, M, r):
    if kind == "grads":
        return grads_algorithmic_bytes(layers, M, r)
    if kind == "fwd":
        return fwd_algorithmic_bytes(layers, M, r)
    if kind == "bwd_dx":
        return bwd_dx_algorithmic_bytes(layers, M, r)
    if kind == "quantize":
        return quantize_algorithmic_bytes(layers)
    d = PMC_DECODE
    return gemv_bytes(d["M"], d["N"], d["K"], d["r"]) - 2 * d["K"] * d["r"]


def measured_traffic(kind):
    """HBM bytes per launch of one GEMM kernel from the committed counter runs, or None when
    they are missing or were taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILES[kind]) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line and not line.startswith("#"))
        if kv.get("source_sha256", "").strip() != gemm_source_sha(kind):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def pmc_summary(fetch_csv, write_csv, kind):
    """Per-launch FETCH_SIZE / WRITE_SIZE of one kernel (fwd, bwd_dx, quantize or gemv), each scaled by
    the factor that makes the same counter read the calibration copy's known bytes."""
    kname = KERNELS[kind]
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(dict)
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] == counter:
                vals[row["Dispatch_Id"]][row["Kernel_Name"]] = vals[row["Dispatch_Id"]].get(row["Kernel_Name"], 0.0) + \
                    float(row["Counter_Value"])
        ker = [v for d in vals.values() for k, v in d.items() if kname in k and (kind != "gemv" or "false>" in k)]
        cal = [v for d in vals.values() for k, v in d.items() if "elementwise" in k]
        if not ker or not cal:
            raise SystemExit(f"{path}: no {kname} or calibration dispatch for {counter}")
        return sum(ker) / len(ker), len(ker), max(cal)

    f_kib, n_f, f_cal = per_kernel(fetch_csv, "FETCH_SIZE")
    w_kib, n_w, w_cal = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = CALIB_BYTES / (f_cal * 1024), CALIB_BYTES / (w_cal * 1024)
    fetch_b, write_b = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
    from bit_nf4_quantized_15_amd import workloads
    cfg = workloads.CONFIGS[workloads.BLOCK_7B]
    algo = algorithmic_bytes(kind, cfg["layers"], cfg["M"], cfg["r"])
    print(f"source_sha256: {gemm_source_sha(kind)}")
    print(f"kernel: {kname}")
    print(f"dispatches: {n_f} (FETCH run), {n_w} (WRITE run)")
    print(f"fetch_kib_per_launch_raw: {f_kib:.1f}")
    print(f"write_kib_per_launch_raw: {w_kib:.1f}")
    print(f"calibration_copy_bytes: {CALIB_BYTES} read + {CALIB_BYTES} written")
    print(f"calibration_fetch_kib: {f_cal:.1f}")
    print(f"calibration_write_kib: {w_cal:.1f}")
    print(f"fetch_scale: {f_scale:.4f}")
    print(f"write_scale: {w_scale:.4f}")
    print(f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"hbm_write_bytes_per_launch: {write_b:.0f}")
    print(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}")
    print(f"algorithmic_bytes_per_launch: {algo:.0f}")
    print(f"traffic_over_algorithmic: {(fetch_b + write_b) / algo:.3f}")


def pmc_decode(torch, qlora, workloads, dev, to_dev, shape, M):
    """Profiler runs of the decode forward on one shape (q_proj, fused q/k/v or fused gate/up, one LoRA
    pair of r = 16 per layer) at M tokens: eight rotated weight copies, each through the layer call
    (t and y in one launch) and through the GEMV kernel for a given t, then the calibration copy."""
    rows, K, r1 = DECODE_SHAPES[shape]
    N, r = sum(rows), r1 * len(rows)
    W = np.concatenate([workloads.custom(9200 + i, (n, K), 0.02) for i, n in enumerate(rows)], axis=0)
    w0 = qlora.quantize(to_dev(W))
    copies = [qlora.NF4Weight(w0.codes.clone(), w0.q8.clone(), w0.a2.clone(), N, K) for _ in range(8)]
    A = to_dev(workloads.custom(9210, (K, r), 0.25))
    B = to_dev(workloads.custom(9220, (r, N), 0.01))
    x = to_dev(workloads.custom(9231, (M, K), 1.0))
    t = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(qlora.fwd_workspace(M, N, K, r), 256), dtype=torch.uint8, device=dev)
    for w in copies:
        qlora.linear_fwd(w, x, A, B, 2.0 * r, y=y, t=t, ws=ws)
    for w in copies:
        qlora.fused_gemm_fwd(w, x, t, B, y=y)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "pmc-decode", "shape": shape, "N": N, "K": K, "r": r, "M": M,
                      "calibration_copy_bytes": CALIB_BYTES}))


def pmc_counters(csv_path):
    """Mean per dispatch of every counter of a rocprofv3 --pmc csv (values of one dispatch summed over
    the rows that carry them), for the path's kernels.  Derived where the counters are there:
    mfma_flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; mfma_busy_share = SQ_VALU_MFMA_BUSY_CYCLES (summed
    over the 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8 (one count per XCD, summed over the 8) x 1024);
    lds_bank_conflict_share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for row in csv.DictReader(open(csv_path)):
        per[row["Dispatch_Id"]][row["Counter_Name"]] += float(row["Counter_Value"])
        names[row["Dispatch_Id"]] = row["Kernel_Name"]
    groups = collections.defaultdict(list)
    for did, vals in per.items():
        kn = names[did]
        for kind, kname in KERNELS.items():
            if kname in kn:
                variant = "t given" if kind == "gemv" and "false>" in kn else ("layer call" if kind == "gemv" else "")
                groups[(kind, variant)].append(vals)
    for (kind, variant), lst in sorted(groups.items()):
        print(f"kernel: {KERNELS[kind]}{' (' + variant + ')' if variant else ''}")
        print(f"dispatches: {len(lst)}")
        counters = sorted({c for v in lst for c in v})
        means = {c: sum(v.get(c, 0.0) for v in lst) / len(lst) for c in counters}
        for c in counters:
            print(f"  {c}: {means[c]:.1f}")
        if means.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            print(f"  mfma_flop: {means['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4e}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in means and means.get("GRBM_GUI_ACTIVE"):
            print(f"  mfma_busy_share: {means['SQ_VALU_MFMA_BUSY_CYCLES'] / (means['GRBM_GUI_ACTIVE'] / 8 * 1024):.4f}")
        if "SQ_LDS_BANK_CONFLICT" in means and means.get("SQ_LDS_IDX_ACTIVE"):
            print(f"  lds_bank_conflict_share: {means['SQ_LDS_BANK_CONFLICT'] / means['SQ_LDS_IDX_ACTIVE']:.4f}")


def layer_flops(M, N, K, r):
    return dict(fwd_gemm=2 * M * K * N + 2 * M * r * N, fwd=2 * M * K * N + 2 * M * r * (K + N),
                bwd_dx_gemm=2 * M * N * K + 2 * M * r * K, bwd=2 * M * K * N + 4 * M * r * (K + N))


def graph_ms(calls, reps=5):
    """Average GPU time per call of `calls`, captured once into a HIP graph and replayed."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls[:2]:
            f()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * len(calls))


def gemv_bytes(M, N, K, r, double_quant=True):
    """Algorithmic HBM bytes of one decode forward: codes, scales (q8 + a2, or the fp32 block absmax
    without double quantization), x, y, A, B."""
    scales = N * K // 64 + 4 * (-(-N * K // 16384)) if double_quant else 4 * (N * K // 64)
    return N * K // 2 + scales + 2 * M * K + 2 * M * N + 2 * K * r + 2 * r * N


def progress(msg):
    """A phase of the run, on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.pmc_kernel)
        return
    if args.pmc_counters:
        pmc_counters(args.pmc_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU and has no collectives: each GPU of a data-parallel job would run it on "
              "its own share of the tokens)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_15_amd import qlora, workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def to_dev(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.mode == "pmc-decode":
        pmc_decode(torch, qlora, workloads, dev, to_dev, args.decode_shape, args.decode_m)
        return

    # ---------------------------------------------------------------- workload: the 7B-like block
    wl = workloads.BLOCK_7B
    cfg = workloads.CONFIGS[wl]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    L = []
    for li, (name, N, K) in enumerate(cfg["layers"]):
        d = dict(name=name, N=N, K=K)
        d["W"] = to_dev(workloads.weight(wl, li))
        d["x"] = to_dev(workloads.activations(wl, li))
        d["A"] = to_dev(workloads.lora_A(wl, li))
        d["B"] = to_dev(workloads.lora_B(wl, li))
        d["dy"] = to_dev(workloads.grad_output(wl, li))
        d["w"] = qlora.NF4Weight.empty(N, K, dev)
        d["t"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        d["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        d["dx"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        d["dA"] = torch.empty((K, r), dtype=torch.float32, device=dev)
        d["dB"] = torch.empty((r, N), dtype=torch.float32, device=dev)
        d["flops"] = layer_flops(M, N, K, r)
        L.append(d)
    ws_bytes = max(max(qlora.bwd_workspace(M, d["N"], d["K"], r), qlora.fwd_workspace(M, d["N"], d["K"], r),
                       int(qlora.lib.qlora_lora_down_workspace(M, d["K"], r))) for d in L)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for d in L:
        d["u"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    grads = [(d["x"], d["t"], d["u"], d["dy"]) for d in L]
    grads_ws = torch.empty(max(1, int(qlora.lib.qlora_lora_grads_batch_workspace(
        (qlora.LoraGrads * len(L))(*[qlora.LoraGrads(0, 0, 0, 0, 0, 0, M, d["N"], d["K"]) for d in L]), len(L), r))),
        dtype=torch.uint8, device=dev)
    total_flops = sum(d["flops"]["fwd"] + d["flops"]["bwd"] for d in L)
    n_weights = sum(d["N"] * d["K"] for d in L)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    timing = dict(fwd_gemm=[], bwd=[], bwd_dx_call=[], grads_batch=[])

    # layers whose inputs are ready together: q, k, v share x, gate and up share theirs (and get their dy
    # together in the backward); o and down wait for the attention and the MLP activation
    groups, cur = [], []
    for i, d in enumerate(L):
        if cur and (L[cur[-1]]["name"], d["name"]) not in SHARED_INPUT:
            groups.append(cur)
            cur = []
        cur.append(i)
    groups.append(cur)
    lw = lambda C: int(qlora.lib.qlora_lora_down_workspace(M, C, r))
    prod_ws = max(max(sum(lw(L[i]["K"]) for i in g), sum(lw(L[i]["N"]) for i in g)) for g in groups)
    if prod_ws > ws.numel():
        ws = torch.empty(prod_ws, dtype=torch.uint8, device=dev)

    def step(record):
        qlora.quantize_batch([d["W"] for d in L], [d["w"] for d in L])
        for g in groups:
            if args.schedule == "grouped":
                qlora.lora_down_batch([(L[i]["x"], L[i]["A"]) for i in g], alpha, t=[L[i]["t"] for i in g], ws=ws)
            for i in g:
                d = L[i]
                if args.schedule != "grouped":
                    qlora.lora_down(d["x"], d["A"], alpha, t=d["t"], ws=ws)
                if record:
                    a = ev(); a.record()
                qlora.fused_gemm_fwd(d["w"], d["x"], d["t"], d["B"], y=d["y"])
                if record:
                    b = ev(); b.record()
                    timing["fwd_gemm"].append((a, b, d["flops"]["fwd_gemm"]))
        if args.schedule == "per-layer":
            for d in L:
                if record:
                    a = ev(); a.record()
                qlora.linear_bwd(d["w"], d["x"], d["A"], d["B"], alpha, d["dy"], t=d["t"], dx=d["dx"], dA=d["dA"],
                                 dB=d["dB"], ws=ws)
                if record:
                    b = ev(); b.record()
                    timing["bwd"].append((a, b, d["flops"]["bwd"]))
            return
        # u and dx (what the layer below waits for) per layer or per group, then the LoRA weight
        # gradients of all layers in one launch
        for g in groups:
            if record:
                a = ev(); a.record()
            if args.schedule == "grouped":
                qlora.lora_u_batch([(L[i]["dy"], L[i]["B"]) for i in g], alpha, u=[L[i]["u"] for i in g], ws=ws)
                for i in g:
                    d = L[i]
                    qlora.fused_gemm_bwd_dx(d["w"], d["dy"], d["u"], d["A"], dx=d["dx"])
            else:
                for i in g:
                    d = L[i]
                    qlora.linear_bwd_dx(d["w"], d["A"], d["B"], alpha, d["dy"], u=d["u"], dx=d["dx"], ws=ws)
            if record:
                b = ev(); b.record()
                timing["bwd_dx_call"].append((a, b, sum(L[i]["flops"]["bwd"] for i in g)))
        if record:
            a = ev(); a.record()
        qlora.lora_grads_batch(grads, dA=[d["dA"] for d in L], dB=[d["dB"] for d in L], ws=grads_ws)
        if record:
            b = ev(); b.record()
            timing["grads_batch"].append((a, b, 0))

    if args.mode == "pmc":
        for _ in range(2):
            step(False)
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)                   # calibration: reads and writes exactly 512 MiB
        torch.cuda.synchronize()
        print(json.dumps({"mode": "pmc", "calibration_copy_bytes": CALIB_BYTES}))
        return

    progress(f"inputs ready; {args.warmup} warmup steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    progress(f"{args.steps} timed steps")
    # the headline: K steps with no events inside (an event recorded between two kernels leaves the GPU
    # idle for several microseconds)
    t_start, t_stop = ev(), ev()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step(False)
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_stop) / args.steps
    value = total_flops / (ms_step * 1e-3) / 1e12
    # the same K steps again with events around each forward GEMM and each backward call, for the breakdown
    progress(f"step {ms_step:.4f} ms ({value:.1f} TFLOP/s); breakdown pass")
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()

    # The step's dominant kernel, the fused backward dx GEMM, on its own: qlora_linear_bwd launches it
    # between other kernels, so it is timed through its stage entry point on the same shapes and inputs.
    # As inside qlora_linear_bwd, each launch follows the kernel that computes u = (alpha/r) dy B^T from
    # dy (untimed here), so dy is as warm in the caches as it is in the step.
    for d in L:
        d["Bt"] = d["B"].t().contiguous()
        d["u"] = qlora.lora_down(d["dy"], d["Bt"], alpha)
    for d in L:
        qlora.fused_gemm_bwd_dx(d["w"], d["dy"], d["u"], d["A"], dx=d["dx"])
    timing["bwd_dx"] = []
    for _ in range(args.steps):
        for d in L:
            qlora.lora_down(d["dy"], d["Bt"], alpha, t=d["u"], ws=ws)
            a = ev(); a.record()
            qlora.fused_gemm_bwd_dx(d["w"], d["dy"], d["u"], d["A"], dx=d["dx"])
            b = ev(); b.record()
            timing["bwd_dx"].append((a, b, d["flops"]["bwd_dx_gemm"]))
    torch.cuda.synchronize()

    def agg(lst):
        tot_ms = sum(a.elapsed_time(b) for a, b, _ in lst)
        tot_f = sum(f for _, _, f in lst)
        return tot_f / (tot_ms * 1e-3) / 1e12, tot_ms / len(lst)

    fwd_tfs, fwd_avg_ms = agg(timing["fwd_gemm"])
    if args.schedule == "per-layer":
        bwd_tfs, bwd_avg_ms = agg(timing["bwd"])
        bwd_sched = {"bwd_schedule": "qlora_linear_bwd per layer"}
    else:
        # a layer's backward: its u and dx and a seventh of the gradient launch
        dx_ms = sum(a.elapsed_time(b) for a, b, _ in timing["bwd_dx_call"])
        gb_ms = sum(a.elapsed_time(b) for a, b, _ in timing["grads_batch"])
        tot_f = sum(f for _, _, f in timing["bwd_dx_call"])
        n_layer_calls = len(timing["grads_batch"]) * len(L)
        bwd_tfs = tot_f / ((dx_ms + gb_ms) * 1e-3) / 1e12
        bwd_avg_ms = (dx_ms + gb_ms) / n_layer_calls
        bwd_sched = {"bwd_schedule": (
                         "per group of layers sharing their input: qlora_lora_u_batch, then qlora_fused_gemm_bwd_dx "
                         "per layer; then qlora_lora_grads_batch over the 7 layers" if args.schedule == "grouped" else
                         "qlora_linear_bwd_dx per layer, then qlora_lora_grads_batch over the 7 layers"),
                     "layer_groups": [[L[i]["name"] for i in g] for g in groups],
                     "u_dx_avg_ms_per_layer": round(dx_ms / n_layer_calls, 4),
                     "lora_grads_batch_ms": round(gb_ms / len(timing["grads_batch"]), 4)}
    bdx_tfs, bdx_avg_ms = agg(timing["bwd_dx"])

    def roofline(kind, tfs, avg_ms, kernel_desc, flop_desc):
        return {"kernel": kernel_desc, "bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": measured_traffic(kind),
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": round(algorithmic_bytes(kind, cfg["layers"], M, r)),
                "avg_launch_ms": round(avg_ms, 4), "per_launch_flop": flop_desc}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded normal weights/activations, no checkpoint)",
        "config": {"workload": cfg["workload"] + " (NF4 quantize + fwd + bwd of all 7 linears)",
                   "M": M, "r": r, "alpha": alpha, "layers": [[d["name"], d["N"], d["K"]] for d in L],
                   "blocksize": 64, "double_quant": "8-bit codes, fp32 per 256 blocks"},
        "roofline": roofline("bwd_dx", bdx_tfs, bdx_avg_ms,
                             "nf4_gemm_bwd_dx_kernel (fused dequant GEMM of dx + LoRA term u A^T; the step's "
                             "largest share of GPU time)",
                             "2*M*N*K + 2*M*r*K over the 7 layer shapes, M=4096, r=64"),
        "breakdown": {"fwd_gemm_roofline": roofline("fwd", fwd_tfs, fwd_avg_ms,
                                                     "nf4_gemm_fwd_kernel (fused dequant GEMM + LoRA up-projection)",
                                                     "2*M*K*N + 2*M*r*N over the 7 layer shapes, M=4096, r=64"),
                      "bwd_call_tflops": round(bwd_tfs, 2), "bwd_call_avg_ms": round(bwd_avg_ms, 4), **bwd_sched,
                      "wall_s_timed": round(wall, 3), "weights_per_step": n_weights,
                      "flop_per_step": total_flops},
    }

    progress(f"backward dx alone {bdx_tfs:.1f} TFLOP/s")
    if not args.no_extras:
        out["extras"] = extras(torch, qlora, workloads, dev, to_dev, L, M, r)
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle on the host)")
        out["cpu_baseline"] = cpu_baseline(workloads, wl, total_flops, n_weights)
    print(json.dumps(out))


def extras(torch, qlora, workloads, dev, to_dev, L, M, r):
    """Decode GEMV bandwidth, quantize/dequantize bandwidth, dense bf16 context."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    res = {}
    # quantize / dequantize of the block's weights (bytes: bf16 in + codes/q8/a2 out)
    q_bytes = sum(d["N"] * d["K"] * 2 + sum(qlora.sizes(d["N"], d["K"])) for d in L)
    for _ in range(2):
        qlora.quantize_batch([d["W"] for d in L], [d["w"] for d in L])
    a, b = ev(), ev()
    a.record()
    reps = 5
    for _ in range(reps):
        qlora.quantize_batch([d["W"] for d in L], [d["w"] for d in L])
    b.record()
    torch.cuda.synchronize()
    q_ms = a.elapsed_time(b) / reps
    res["quantize"] = {"GB/s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "ms": round(q_ms, 4),
                       "frac_of_hbm_peak": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "weights": sum(d["N"] * d["K"] for d in L)}
    d0 = L[0]
    out = torch.empty((d0["N"], d0["K"]), dtype=torch.bfloat16, device=dev)
    qlora.dequantize(d0["w"], out=out)
    a, b = ev(), ev()
    a.record()
    for _ in range(reps):
        qlora.dequantize(d0["w"], out=out)
    b.record()
    torch.cuda.synchronize()
    dq_ms = a.elapsed_time(b) / reps
    dq_bytes = d0["N"] * d0["K"] * 2 + sum(qlora.sizes(d0["N"], d0["K"]))
    res["dequantize_q_proj"] = {"GB/s": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1), "ms": round(dq_ms, 4)}
    del out

    progress("extras: decode")
    res["decode"] = extras_decode(torch, qlora, workloads, dev, to_dev)

    progress("extras: up_proj M=2048, 70B MLP M=8192")
    res["up_proj_M2048_fwd_bwd"] = extras_train(torch, qlora, workloads, dev, to_dev, workloads.UP_PROJ_M2048, 10)
    res["mlp_70b_M8192_fwd_bwd"] = extras_train(torch, qlora, workloads, dev, to_dev, workloads.MLP_70B, 3)
    progress("extras: double quant off, fp4, fp16, pooled, fp32")
    res["double_quant_off"] = extras_variant(torch, qlora, workloads, dev, to_dev, L, M, r, ev, double_quant=False)
    res["fp4"] = extras_variant(torch, qlora, workloads, dev, to_dev, L, M, r, ev, quant_type="fp4")
    res["fp16_compute"] = extras_variant(torch, qlora, workloads, dev, to_dev, L, M, r, ev, dtype=torch.float16)
    res["qa_lora_pooled_g64"] = extras_pooled(torch, qlora, workloads, dev, to_dev, L, M, r, ev, 64)
    res["fp32_compute"] = extras_fp32(torch, qlora, workloads, dev, L, M, r, ev)

    # LoRA merge for deployment (qlora_merge) of the 7 layers: N*K*r fp32 FMAs (VALU-bound) and
    # codes + scales + A + B in, the bf16 merged weight out
    mo = [torch.empty((d["N"], d["K"]), dtype=torch.bfloat16, device=dev) for d in L]
    for d, o in zip(L, mo):
        qlora.merge(d["w"], d["A"], d["B"], workloads.CONFIGS[workloads.BLOCK_7B]["alpha"], out=o)
    a, b = ev(), ev()
    a.record()
    for _ in range(reps):
        for d, o in zip(L, mo):
            qlora.merge(d["w"], d["A"], d["B"], workloads.CONFIGS[workloads.BLOCK_7B]["alpha"], out=o)
    b.record()
    torch.cuda.synchronize()
    m_ms = a.elapsed_time(b) / reps
    m_bytes = sum(sum(qlora.sizes(d["N"], d["K"])) + 2 * r * (d["N"] + d["K"]) + 2 * d["N"] * d["K"] for d in L)
    m_fma = sum(d["N"] * d["K"] * r for d in L)
    res["merge"] = {"ms": round(m_ms, 4), "GB/s": round(m_bytes / (m_ms * 1e-3) / 1e9, 1),
                    "tera_fma_per_s": round(m_fma / (m_ms * 1e-3) / 1e12, 2),
                    "frac_of_fp32_vector_fma_peak": round(m_fma / (m_ms * 1e-3) / (FP32_VECTOR_PEAK_TFS * 1e12 / 2), 4)}
    del mo

    # context: dense bf16 torch.matmul (hipBLASLt) on the same shapes, forward base product only
    tot_f, tot_ms = 0, 0.0
    for d in L:
        Wd = d["W"]
        torch.matmul(d["x"], Wd.t())
        a, b = ev(), ev()
        a.record()
        for _ in range(3):
            torch.matmul(d["x"], Wd.t())
        b.record()
        torch.cuda.synchronize()
        tot_ms += a.elapsed_time(b) / 3
        tot_f += 2 * M * d["N"] * d["K"]
    res["context_dense_bf16_matmul_fwd_tflops"] = round(tot_f / (tot_ms * 1e-3) / 1e12, 1)
    return res


def plain_read_us(torch, qlora, nbytes, dev):
    """Same-size ceiling for a decode launch: the library's plain-read probe (qlora_read_probe, coalesced
    16-byte loads and nothing else) over nbytes, the faster of its two launch shapes, over buffers
    rotated past the 256 MB Infinity Cache, replayed from a HIP graph."""
    n = max(4, -(-600_000_000 // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(n)]
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    best = None
    for variant in (0, 1):
        ms = graph_ms([lambda b=b: qlora.read_probe(b, sink, variant) for b in bufs])
        best = ms if best is None else min(best, ms)
    del bufs
    return best * 1e3


def extras_decode(torch, qlora, workloads, dev, to_dev):
    """Decode forward (M = 1 and 16 tokens) on three weights: the 4096x4096 q_proj (r = 16, 0.1 % outliers)
    and fused q/k/v (3x4096x4096) and gate/up (2x11008x4096) weights.  q/k/v (and gate/up) read the same x,
    so their weights concatenated along N are one NF4 weight (K = 4096: a row holds 64 blocks and a scale
    group 4 rows, so no group spans two layers and the codes and scales equal those of the separate
    weights).  Each layer keeps its own r = 16 LoRA pair: A concatenated along r, B block-diagonal (its zero
    blocks add exact zeros).  For each: the layer call qlora_linear_fwd (t = s x A and y in one launch), the
    GEMV kernel alone for a given t (qlora_fused_gemm_fwd), and a plain read of the kernel's bytes as the
    same-size ceiling.  Weight copies rotated past the 256 MB Infinity Cache, launches replayed from a HIP
    graph (GPU time per call without host launch latency)."""
    out = {}
    K, r1 = 4096, 16
    qd = workloads.CONFIGS[workloads.Q_PROJ_DECODE]
    shapes = (("q_proj_4096x4096_r16", [4096], None), ("qkv_3x4096x4096", [4096, 4096, 4096], 9100),
              ("gate_up_2x11008x4096", [11008, 11008], 9200))
    for name, Ns, seed in shapes:
        N, r = sum(Ns), r1 * len(Ns)
        if seed is None:      # the q_proj decode config itself
            W = workloads.weight(workloads.Q_PROJ_DECODE)
            A = to_dev(workloads.lora_A(workloads.Q_PROJ_DECODE))
            Bbd = to_dev(workloads.lora_B(workloads.Q_PROJ_DECODE))
            alpha = qd["alpha"]
        else:
            W = np.concatenate([workloads.custom(seed + i, (n, K), 0.02) for i, n in enumerate(Ns)], axis=0)
            A = to_dev(np.concatenate([workloads.custom(seed + 10 + i, (K, r1), 0.25) for i in range(len(Ns))],
                                      axis=1))
            Bbd = torch.zeros((r, N), dtype=torch.bfloat16, device=dev)
            n0 = 0
            for i, n in enumerate(Ns):
                Bbd[r1 * i:r1 * (i + 1), n0:n0 + n] = to_dev(workloads.custom(seed + 20 + i, (r1, n), 0.01))
                n0 += n
            alpha = 2.0 * r
        w0 = qlora.quantize(to_dev(W))
        del W
        ncopy = max(4, -(-600_000_000 // (N * K // 2)))
        copies = [qlora.NF4Weight(w0.codes.clone(), w0.q8.clone(), w0.a2.clone(), N, K) for _ in range(ncopy)]
        res = {}
        for Md in (1, 16):
            xd = to_dev(workloads.activations(workloads.Q_PROJ_DECODE, M=Md)) if seed is None else \
                to_dev(workloads.custom(seed + 30 + Md, (Md, K), 1.0))
            td = torch.empty((Md, r), dtype=torch.bfloat16, device=dev)
            yd = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(qlora.fwd_workspace(Md, N, K, r), 256), dtype=torch.uint8, device=dev)
            for w in copies[:4]:
                qlora.linear_fwd(w, xd, A, Bbd, alpha, y=yd, t=td, ws=ws)
            torch.cuda.synchronize()
            k_ms = graph_ms([lambda w=w: qlora.fused_gemm_fwd(w, xd, td, Bbd, y=yd) for w in copies])
            c_ms = graph_ms([lambda w=w: qlora.linear_fwd(w, xd, A, Bbd, alpha, y=yd, t=td, ws=ws) for w in copies])
            nb_call = gemv_bytes(Md, N, K, r)
            nb_kernel = nb_call - 2 * K * r        # A is read by the call's producers, not by the GEMV tiles
            ceil_us = plain_read_us(torch, qlora, nb_call, dev)
            res[f"M={Md}"] = {
                "fwd_call_us": round(c_ms * 1e3, 2), "gemv_kernel_us": round(k_ms * 1e3, 2),
                "call_over_kernel": round(c_ms / k_ms, 3),
                "bytes_fwd_call": nb_call, "bytes_gemv_kernel": nb_kernel,
                "GB/s_fwd_call": round(nb_call / (c_ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak_fwd_call": round(nb_call / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "GB/s_gemv_kernel": round(nb_kernel / (k_ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak_gemv_kernel": round(nb_kernel / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "plain_read_same_bytes_us": round(ceil_us, 2),
                "GB/s_plain_read_same_bytes": round(nb_call / (ceil_us * 1e-6) / 1e9, 1),
                "fwd_call_over_plain_read": round(c_ms * 1e3 / ceil_us, 3)}
        out[name] = res
        del copies, w0
    return out


def extras_train(torch, qlora, workloads, dev, to_dev, wl, steps):
    """Forward + backward of every layer of a training config (the up_proj config, M = 2048, and the
    70B-like MLP, M = 8192): TFLOP/s over the same algorithmic FLOP as the headline (2MKN forward base,
    2MKN dx, 6Mr(K+N) LoRA), weights already quantized; for the 70B MLP also the quantize rate of its
    704.6M weights (bf16 in, codes + q8 + a2 out) against HBM peak."""
    cfg = workloads.CONFIGS[wl]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    L = []
    for li, (name, N, K) in enumerate(cfg["layers"]):
        d = dict(N=N, K=K)
        d["W"] = to_dev(workloads.weight(wl, li))
        d["x"] = to_dev(workloads.activations(wl, li))
        d["A"] = to_dev(workloads.lora_A(wl, li))
        d["B"] = to_dev(workloads.lora_B(wl, li))
        d["dy"] = to_dev(workloads.grad_output(wl, li))
        d["w"] = qlora.quantize(d["W"])
        d["t"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        d["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        d["dx"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        d["dA"] = torch.empty((K, r), dtype=torch.float32, device=dev)
        d["dB"] = torch.empty((r, N), dtype=torch.float32, device=dev)
        L.append(d)
    ws = torch.empty(max(max(qlora.bwd_workspace(M, d["N"], d["K"], r), qlora.fwd_workspace(M, d["N"], d["K"], r))
                         for d in L), dtype=torch.uint8, device=dev)
    for d in L:
        d["u"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    flops = sum(4 * M * d["N"] * d["K"] + 6 * M * r * (d["N"] + d["K"]) for d in L)

    groups, cur = [], []
    for i, (name, _, _) in enumerate(cfg["layers"]):
        if cur and (cfg["layers"][cur[-1]][0], name) not in SHARED_INPUT:
            groups.append(cur)
            cur = []
        cur.append(i)
    groups.append(cur)
    lw = lambda C: int(qlora.lib.qlora_lora_down_workspace(M, C, r))
    prod_ws = max(max(sum(lw(L[i]["K"]) for i in g), sum(lw(L[i]["N"]) for i in g)) for g in groups)
    if prod_ws > ws.numel():
        ws = torch.empty(prod_ws, dtype=torch.uint8, device=dev)

    def step():
        # the headline's grouped schedule: t and u per group of layers that share their input, the GEMMs
        # per layer, then the LoRA weight gradients of all layers in one launch
        for g in groups:
            qlora.lora_down_batch([(L[i]["x"], L[i]["A"]) for i in g], alpha, t=[L[i]["t"] for i in g], ws=ws)
            for i in g:
                qlora.fused_gemm_fwd(L[i]["w"], L[i]["x"], L[i]["t"], L[i]["B"], y=L[i]["y"])
        for g in groups:
            qlora.lora_u_batch([(L[i]["dy"], L[i]["B"]) for i in g], alpha, u=[L[i]["u"] for i in g], ws=ws)
            for i in g:
                qlora.fused_gemm_bwd_dx(L[i]["w"], L[i]["dy"], L[i]["u"], L[i]["A"], dx=L[i]["dx"])
        qlora.lora_grads_batch([(d["x"], d["t"], d["u"], d["dy"]) for d in L], dA=[d["dA"] for d in L],
                               dB=[d["dB"] for d in L])

    for _ in range(2):
        step()
    a, b = ev(), ev()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    res = {"layers": [[n, N, K] for n, N, K in cfg["layers"]], "M": M, "r": r, "steps": steps,
           "fwd_bwd_ms": round(ms, 4), "fwd_bwd_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}
    if wl == workloads.MLP_70B:
        qlora.quantize_batch([d["W"] for d in L], [d["w"] for d in L])
        a, b = ev(), ev()
        a.record()
        for _ in range(steps):
            qlora.quantize_batch([d["W"] for d in L], [d["w"] for d in L])
        b.record()
        torch.cuda.synchronize()
        q_ms = a.elapsed_time(b) / steps
        q_bytes = sum(d["N"] * d["K"] * 2 + sum(qlora.sizes(d["N"], d["K"])) for d in L)
        res["quantize"] = {"weights": sum(d["N"] * d["K"] for d in L), "ms": round(q_ms, 4),
                           "GB/s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del L, ws
    torch.cuda.empty_cache()
    return res


def extras_fp32(torch, qlora, workloads, dev, L, M, r, ev):
    """The fp32 compute dtype (deep dive 8.3) on the same 7 linears: every tensor fp32 (the bf16 draws
    widened exactly), w_hat = fl32(a_hat * c_q), products on the fp32 matrix cores.  The whole quantize +
    fwd + bwd step and the forward call, against the 157.3 TFLOP/s dense fp32 MFMA peak."""
    alpha = workloads.CONFIGS[workloads.BLOCK_7B]["alpha"]
    f = torch.float32
    Lf = [dict(N=d["N"], K=d["K"], flops=d["flops"], W=d["W"].to(f), x=d["x"].to(f), A=d["A"].to(f),
               B=d["B"].to(f), dy=d["dy"].to(f), t=torch.empty((M, r), dtype=f, device=dev),
               y=torch.empty((M, d["N"]), dtype=f, device=dev), dx=torch.empty((M, d["K"]), dtype=f, device=dev),
               dA=d["dA"], dB=d["dB"]) for d in L]
    Wn = [qlora.NF4Weight.empty(d["N"], d["K"], dev, dtype=f) for d in Lf]
    ws = torch.empty(max(max(qlora.bwd_workspace(M, d["N"], d["K"], r, f), qlora.fwd_workspace(M, d["N"], d["K"], r, f))
                         for d in Lf), dtype=torch.uint8, device=dev)
    total_flops = sum(d["flops"]["fwd"] + d["flops"]["bwd"] for d in Lf)
    fwd_flops = sum(d["flops"]["fwd"] for d in Lf)

    def fwd():
        for d, w in zip(Lf, Wn):
            qlora.linear_fwd(w, d["x"], d["A"], d["B"], alpha, y=d["y"], t=d["t"], ws=ws)

    def step():
        for d, w in zip(Lf, Wn):
            qlora.quantize(d["W"], out=w)
        fwd()
        for d, w in zip(Lf, Wn):
            qlora.linear_bwd(w, d["x"], d["A"], d["B"], alpha, d["dy"], t=d["t"], dx=d["dx"], dA=d["dA"],
                             dB=d["dB"], ws=ws)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    step_ms = timed(step, 3)
    fwd_ms = timed(fwd, 3)
    step_tfs = total_flops / (step_ms * 1e-3) / 1e12
    fwd_tfs = fwd_flops / (fwd_ms * 1e-3) / 1e12
    del Lf, Wn, ws
    return {"step": {"ms": round(step_ms, 3), "TFLOP/s": round(step_tfs, 2),
                     "frac_of_fp32_mfma_peak": round(step_tfs / MFMA_F32_PEAK_TFS, 4)},
            "fwd_call": {"ms_7_layers": round(fwd_ms, 3), "TFLOP/s": round(fwd_tfs, 2),
                         "frac_of_fp32_mfma_peak": round(fwd_tfs / MFMA_F32_PEAK_TFS, 4)}}


def extras_variant(torch, qlora, workloads, dev, to_dev, L, M, r, ev, double_quant=True, quant_type="nf4",
                   dtype=None):
    """The same workloads with another scale layout, codebook or compute dtype: double quantization off
    (fp32 absmax per block, deep dive 7.1 and 9.5), the fp4 codebook (deep dive 6.5, 8.1) or fp16 compute
    (deep dive 8.3; the same draws rounded to fp16).  The whole quantize + fwd + bwd step of the 7 linears,
    the forward GEMM alone, quantize bandwidth and the decode GEMV (64 rotated weight copies)."""
    res = {}
    alpha = workloads.CONFIGS[workloads.BLOCK_7B]["alpha"]
    dt = torch.bfloat16 if dtype is None else dtype
    if dt != torch.bfloat16:
        L = [dict(d, W=d["W"].to(dt), x=d["x"].to(dt), A=d["A"].to(dt), B=d["B"].to(dt), dy=d["dy"].to(dt),
                  t=torch.empty_like(d["t"], dtype=dt), y=torch.empty_like(d["y"], dtype=dt),
                  dx=torch.empty_like(d["dx"], dtype=dt)) for d in L]
    Wn = [qlora.NF4Weight.empty(d["N"], d["K"], dev, double_quant=double_quant, quant_type=quant_type, dtype=dt)
          for d in L]
    ws = torch.empty(max(qlora.bwd_workspace(M, d["N"], d["K"], r) for d in L), dtype=torch.uint8, device=dev)
    total_flops = sum(d["flops"]["fwd"] + d["flops"]["bwd"] for d in L)
    fwd_flops = sum(d["flops"]["fwd_gemm"] for d in L)

    def quant():
        qlora.quantize_batch([d["W"] for d in L], Wn)

    def fwd():
        for d, w in zip(L, Wn):
            qlora.fused_gemm_fwd(w, d["x"], d["t"], d["B"], y=d["y"])

    def step():
        quant()
        for d, w in zip(L, Wn):
            qlora.lora_down(d["x"], d["A"], alpha, t=d["t"], ws=ws)
            qlora.fused_gemm_fwd(w, d["x"], d["t"], d["B"], y=d["y"])
        for d, w in zip(L, Wn):
            qlora.linear_bwd(w, d["x"], d["A"], d["B"], alpha, d["dy"], t=d["t"], dx=d["dx"], dA=d["dA"],
                             dB=d["dB"], ws=ws)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    step_ms = timed(step, 5)
    fwd_ms = timed(fwd, 5)
    q_ms = timed(quant, 5)
    size_of = qlora.sizes if double_quant else qlora.sizes_nodq
    q_bytes = sum(d["N"] * d["K"] * 2 + sum(size_of(d["N"], d["K"])) for d in L)
    res["step"] = {"ms": round(step_ms, 4), "TFLOP/s": round(total_flops / (step_ms * 1e-3) / 1e12, 2)}
    res["fwd_gemm"] = {"avg_launch_ms": round(fwd_ms / len(L), 4),
                       "TFLOP/s": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2)}
    res["quantize"] = {"GB/s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "ms": round(q_ms, 4),
                       "bytes_per_weight": round(q_bytes / sum(d["N"] * d["K"] for d in L), 4)}
    del Wn, ws, L
    qd = workloads.CONFIGS[workloads.Q_PROJ_DECODE]
    _, N2, K2 = qd["layers"][0]
    W2 = to_dev(workloads.weight(workloads.Q_PROJ_DECODE)).to(dt)
    copies = [qlora.quantize(W2, double_quant=double_quant, quant_type=quant_type) for _ in range(64)]
    B2 = to_dev(workloads.lora_B(workloads.Q_PROJ_DECODE)).to(dt)
    xd = to_dev(workloads.activations(workloads.Q_PROJ_DECODE, M=1)).to(dt)
    td = torch.zeros((1, qd["r"]), dtype=dt, device=dev)
    yd = torch.empty((1, N2), dtype=dt, device=dev)
    for w in copies[:4]:
        qlora.fused_gemm_fwd(w, xd, td, B2, y=yd)
    torch.cuda.synchronize()
    gemv_ms = graph_ms([lambda w=w: qlora.fused_gemm_fwd(w, xd, td, B2, y=yd) for w in copies])
    nb = gemv_bytes(1, N2, K2, qd["r"], double_quant=double_quant) - 2 * K2 * qd["r"]
    res["decode_gemv_q_proj_M=1"] = {"gemv_kernel_us": round(gemv_ms * 1e3, 2), "bytes_gemv_kernel": nb,
                                     "GB/s_gemv_kernel": round(nb / (gemv_ms * 1e-3) / 1e9, 1)}
    return res


def extras_pooled(torch, qlora, workloads, dev, to_dev, L, M, r, ev, g):
    """The whole quantize + fwd + bwd step of the 7 linears with the QA-LoRA pooled branch
    ("LoRA, QLoRA, QA-LoRA explained", sections 3-5): A is [K/g, r] and the LoRA input is the mean
    of each group of g columns of x.  Reported beside the plain step it replaces."""
    alpha = workloads.CONFIGS[workloads.BLOCK_7B]["alpha"]
    Ap = [to_dev(workloads.custom(900 + i, (d["K"] // g, r), float(1 / np.sqrt(r)))) for i, d in enumerate(L)]
    ws = torch.empty(max(max(qlora.lib.qlora_pooled_fwd_workspace(M, d["N"], d["K"], r, g),
                              qlora.lib.qlora_pooled_bwd_workspace(M, d["N"], d["K"], r, g)) for d in L),
                     dtype=torch.uint8, device=dev)
    dAp = [torch.empty((d["K"] // g, r), dtype=torch.float32, device=dev) for d in L]

    def step():
        for d in L:
            qlora.quantize(d["W"], out=d["w"])
        for d, A in zip(L, Ap):
            qlora.pooled_fwd(d["w"], d["x"], A, d["B"], alpha, g, y=d["y"], t=d["t"], ws=ws)
        for d, A, dA in zip(L, Ap, dAp):
            qlora.pooled_bwd(d["w"], d["x"], A, d["B"], alpha, g, d["dy"], t=d["t"], dx=d["dx"], dA=dA, dB=d["dB"],
                             ws=ws)

    step()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    reps = 5
    for _ in range(reps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    total_flops = sum(d["flops"]["fwd"] + d["flops"]["bwd"] for d in L)
    return {"g": g, "step_ms": round(ms, 4), "TFLOP/s_plain_step_flops": round(total_flops / (ms * 1e-3) / 1e12, 2)}


def cpu_baseline(workloads, wl, total_flops, n_weights):
    """The oracle as it stands, on the host cores, on a bounded sample of the same step:
    quantize two of the seven weights (q_proj, gate_proj) and run fp64 forward+backward
    on 256 of the 4096 token rows for those two layers; the full-step time is
    extrapolated from the measured quantize rate (weights/s) and fp64 GEMM rate (FLOP/s)."""
    from oracle import bf16, lora, nf4
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    cfg = workloads.CONFIGS[wl]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    rows = 256
    q_w, q_s, f_f, f_s = 0, 0.0, 0, 0.0
    for li in (0, 4):
        name, N, K = cfg["layers"][li]
        W = workloads.weight(wl, li)
        t0 = time.perf_counter()
        p, q8, a2 = nf4.quantize(W)
        q_s += time.perf_counter() - t0
        q_w += N * K
        x = workloads.activations(wl, li)[:rows]
        dy = workloads.grad_output(wl, li)[:rows]
        A = workloads.lora_A(wl, li); B = workloads.lora_B(wl, li)
        t0 = time.perf_counter()
        Wh = bf16.to_f64(nf4.dequantize(p, q8, a2, N, K))
        xf, Af, Bf, dyf = (bf16.to_f64(v) for v in (x, A, B, dy))
        lora.linear_fwd(xf, Wh, Af, Bf, alpha, r)
        lora.linear_bwd(xf, Wh, Af, Bf, alpha, r, dyf)
        f_s += time.perf_counter() - t0
        f_f += 4 * rows * K * N + 6 * rows * r * (K + N)
    est_s = n_weights / (q_w / q_s) + total_flops / (f_f / f_s)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"value": round(total_flops / est_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "cpu_model": cpu_model, "nproc": os.cpu_count(), "usable_cpus": usable,
            "kind": "oracle",
            "sample": (f"numpy fp64 oracle: quantize q_proj+gate_proj ({q_w} weights, {q_s:.1f} s, 1 thread) and "
                       f"fwd+bwd on {rows}/{M} token rows of those layers ({f_f / 1e9:.1f} GFLOP, {f_s:.1f} s, "
                       f"BLAS threads {blas_threads}); full step extrapolated to {est_s:.1f} s"),
            "sample_seconds": round(q_s + f_s, 2)}


if __name__ == "__main__":
    main()
