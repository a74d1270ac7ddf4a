"""Host-side checks of bench.py's accounting (no GPU needed).

* the FLOP count of a step is the sum of the layer's contractions, restated
  here product by product;
* the algorithmic bytes of the GEMM launches and of the decode GEMV are the
  tensor sizes the kernels must move, restated here tensor by tensor;
* the counter summary scales FETCH_SIZE / WRITE_SIZE by what the same counter
  reads for the calibration copy, and sums a dispatch's per-instance rows;
* the recorded HBM traffic is reported only while the GEMM source (comments
  aside) is the one it was measured on;
* --gpus N for N other than 1 exits with a message before touching a GPU.
"""
import os
import subprocess
import sys

import pytest

import bench
from bit_nf4_quantized_15_amd import workloads

BLOCK = workloads.CONFIGS[workloads.BLOCK_7B]


def test_step_flops_are_the_sum_of_the_contractions():
    M, r = BLOCK["M"], BLOCK["r"]
    total = 0
    for _, N, K in BLOCK["layers"]:
        forward = 2 * M * K * N + 2 * M * K * r + 2 * M * r * N          # x W^T, x A, t B
        backward = (2 * M * N * K + 2 * M * N * r + 2 * M * r * K          # dy W, dy B^T, u A^T
                    + 2 * K * M * r + 2 * r * M * N)                       # x^T u, t^T dy
        f = bench.layer_flops(M, N, K, r)
        assert f["fwd"] == forward and f["bwd"] == backward
        assert f["fwd_gemm"] == 2 * M * K * N + 2 * M * r * N
        assert f["bwd_dx_gemm"] == 2 * M * N * K + 2 * M * r * K
        total += forward + backward
    assert total == 3438523973632                                          # 3.4385 TFLOP per step


def test_gemm_algorithmic_bytes_are_the_tensor_sizes():
    M, r = BLOCK["M"], BLOCK["r"]
    fwd, bwd = [], []
    for _, N, K in BLOCK["layers"]:
        codes, q8, a2 = N * K // 2, N * K // 64, 4 * ((N * K + 16383) // 16384)
        fwd.append(M * K * 2 + codes + q8 + a2 + M * r * 2 + r * N * 2 + M * N * 2)     # x, w, t, B in; y out
        bwd.append(M * N * 2 + codes + q8 + a2 + M * r * 2 + K * r * 2 + M * K * 2)     # dy, w, u, A in; dx out
    assert bench.algorithmic_bytes("fwd", BLOCK["layers"], M, r) == pytest.approx(sum(fwd) / 7, rel=1e-12)
    assert bench.algorithmic_bytes("bwd_dx", BLOCK["layers"], M, r) == pytest.approx(sum(bwd) / 7, rel=1e-12)
    assert round(sum(bwd) / 7) == 107465033
    grads = sum(M * K * 2 + M * N * 2 + M * r * 2 * 2 + K * r * 4 + r * N * 4      # x, dy, u, t in; dA, dB out
                for _, N, K in BLOCK["layers"])
    assert bench.algorithmic_bytes("grads", BLOCK["layers"], M, r) == grads


def test_decode_gemv_bytes_of_q_proj():
    N = K = 4096
    r = 16
    codes, q8, a2 = N * K // 2, N * K // 64, 4 * (N * K // 16384)
    for M in (1, 16):
        want = codes + q8 + a2 + M * K * 2 + M * N * 2 + K * r * 2 + r * N * 2     # + A for the whole call
        assert bench.gemv_bytes(M, N, K, r) == want
    assert bench.gemv_bytes(1, N, K, r) - 2 * K * r == 8802304                     # the GEMV kernel alone
    nodq = N * K // 2 + 4 * (N * K // 64) + K * 2 + N * 2 + K * r * 2 + r * N * 2
    assert bench.gemv_bytes(1, N, K, r, double_quant=False) == nodq


def _write_counter_csv(path, counter, dispatches):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did, name, values in dispatches:
            for v in values:                                                # one row per counter instance
                f.write(f'{did},"{name}",{counter},{v}\n')


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path, capsys):
    kern = "void qlora::(anonymous namespace)::nf4_gemm_bwd_dx_kernel<true, true, 0, 0>(...)"
    cal = "void at::native::elementwise_kernel<128, 4>(...)"
    calib_kib = bench.CALIB_BYTES // 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # FETCH_SIZE reads half of the calibration's bytes, WRITE_SIZE all of them
    _write_counter_csv(fetch, "FETCH_SIZE", [(1, kern, [1000.0, 1000.0]), (2, kern, [1500.0, 1500.0]),
                                             (3, cal, [calib_kib / 4, calib_kib / 4])])
    _write_counter_csv(write, "WRITE_SIZE", [(1, kern, [400.0]), (2, kern, [600.0]), (3, cal, [calib_kib])])
    bench.pmc_summary(str(fetch), str(write), "bwd_dx")
    out = dict(line.split(": ", 1) for line in capsys.readouterr().out.splitlines() if ": " in line)
    assert float(out["fetch_scale"]) == pytest.approx(2.0)
    assert float(out["write_scale"]) == pytest.approx(1.0)
    assert float(out["hbm_fetch_bytes_per_launch"]) == pytest.approx(2500.0 * 1024 * 2.0, abs=1)
    assert float(out["hbm_write_bytes_per_launch"]) == pytest.approx(500.0 * 1024, abs=1)
    assert out["dispatches"].startswith("2 ")


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.txt"
    monkeypatch.setitem(bench.TRAFFIC_FILES, "bwd_dx", str(rec))
    rec.write_text(f"# header\nsource_sha256: {bench.gemm_source_sha('bwd_dx')}\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("bwd_dx") == 123456.0
    rec.write_text("source_sha256: " + "0" * 64 + "\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("bwd_dx") is None                       # taken on other code
    rec.unlink()
    assert bench.measured_traffic("bwd_dx") is None                       # no record
    # each kind hashes its own source: the GEMMs gemm.hip, quantize quantize.hip, the GEMV gemv.hip
    assert bench.gemm_source_sha("fwd") == bench.gemm_source_sha("bwd_dx") != bench.gemm_source_sha("gemv")
    # comments do not change the hash; code does
    src = open(os.path.join(bench._CSRC, bench.SOURCES["bwd_dx"])).read()
    sha = bench.gemm_source_sha("bwd_dx")
    monkeypatch.setattr(bench, "_CSRC", str(tmp_path))
    copy = tmp_path / bench.SOURCES["bwd_dx"]
    copy.write_text("// a new comment\n" + src.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.gemm_source_sha("bwd_dx") == sha
    copy.write_text(src + "\nint extra_symbol;\n")
    assert bench.gemm_source_sha("bwd_dx") != sha


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(bench.HERE, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
