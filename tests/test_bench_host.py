"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
algorithmic byte counts behind the roofline figures, and the parsing and
scaling of rocprofv3 counter files into the profile summaries."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_dit_shapes():
    # MLP up, int4 g64, rank 32: codes of both operands in the FP6 layout (48
    # bytes per 64 codes), one bf16 scale per 64 codes, fp32 lora_act, bf16
    # lora_up, bf16 out
    M, N, K, r = 4096, 12288, 3072, 32
    want = (M + N) * K * 3 // 4 + (M + N) * (K // 64) * 2 + M * r * 4 + N * r * 2 + M * N * 2
    assert want == 141295616
    assert bench.algorithmic_bytes_gemm(M, N, K, r, "int4") == want
    # NVFP4: one E4M3 byte per 16 codes instead
    assert bench.algorithmic_bytes_gemm(4096, 3072, 3072, 32, "nvfp4") == \
        7168 * 1536 + 7168 * 192 + 4096 * 128 + 3072 * 64 + 4096 * 3072 * 2
    # quantize: bf16 x in, codes + scales + fp32 t out, smooth and L1 read once
    assert bench.algorithmic_bytes_quantize(4096, 3072, 32, "int4") == \
        4096 * 3072 * 2 + 3072 * 2 + 32 * 3072 * 2 + 4096 * 2304 + 4096 * 48 * 2 + 4096 * 32 * 4
    # adaLN GEMV at M = 1: 18432 x 3072 int4 codes, bf16 scales and zero points per 64
    assert bench.algorithmic_bytes_gemv(1, 18432, 3072) == 31893504


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_means_sum_dimensions_and_average_dispatches(tmp_path):
    k = "void svdq::gemm_w4a4_int4_kernel<false, true, false>(int, ...)"
    # two dispatches; SQ_INSTS_VALU reported per shader engine (two rows each)
    _write_counters(str(tmp_path / "r"), [
        (1, k, "SQ_INSTS_VALU", 10), (1, k, "SQ_INSTS_VALU", 30), (1, k, "MfmaUtil", 35.0),
        (2, k, "SQ_INSTS_VALU", 20), (2, k, "SQ_INSTS_VALU", 40), (2, k, "MfmaUtil", 37.0),
        (3, "__amd_rocclr_copyBuffer", "SQ_INSTS_VALU", 999),
    ])
    m = bench._counter_means(str(tmp_path / "r"), "gemm_w4a4_int4")
    assert m["SQ_INSTS_VALU"] == (50.0, 2)
    assert m["MfmaUtil"] == (36.0, 2)
    with pytest.raises(SystemExit):
        bench._counter_means(str(tmp_path / "r"), "no_such_kernel")


def test_utilisation_and_gemv_traffic_summaries(tmp_path, monkeypatch):
    run = tmp_path / "run"
    g = "void svdq::gemm_w4a4_fp6_kernel<false, true, false>(int, ...)"
    v = "void svdq::awq_gemv_kernel<2, true>(int, ...)"
    c = "__amd_rocclr_copyBuffer"
    _write_counters(str(run / "pmc_gemm_util"), [(1, g, "MfmaUtil", 35.5), (1, g, "VALUBusy", 72.0)])
    wg = (4096 // 64) * (12288 // 64) * (3072 // 64)
    _write_counters(str(run / "pmc_gemm_insts"), [
        (1, g, "SQ_INSTS_VALU", 200 * wg), (1, g, "SQ_INSTS_MFMA", 10 * wg), (1, g, "SQ_INSTS_LDS", 1),
        (1, g, "SQ_INSTS_SALU", 1), (1, g, "SQ_WAVES", 12288)])
    # the copy reads report half the bytes (factor 2), writes all of them
    _write_counters(str(run / "pmc_copy_FETCH_SIZE"), [(1, c, "FETCH_SIZE", 128 * 1024)])
    _write_counters(str(run / "pmc_copy_WRITE_SIZE"), [(1, c, "WRITE_SIZE", 256 * 1024)])
    _write_counters(str(run / "pmc_gemv_FETCH_SIZE"), [(1, v, "FETCH_SIZE", 15625.0), (2, v, "FETCH_SIZE", 15625.0)])
    _write_counters(str(run / "pmc_gemv_WRITE_SIZE"), [(1, v, "WRITE_SIZE", 36.0)])
    # GRBM_GUI_ACTIVE sums the XCDs' active cycles: divided by the agent's XCD count
    _write_counters(str(run / "pmc_gemm_clock"), [(1, g, "GRBM_GUI_ACTIVE", 2400000.0), (1, g, "SQ_BUSY_CYCLES", 1)])
    with open(run / "pmc_gemm_clock" / "run_agent_info.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Node_Id", "Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Node_Id": 0, "Agent_Type": "CPU", "Num_Xcc": 1})
        w.writerow({"Node_Id": 1, "Agent_Type": "GPU", "Num_Xcc": 8})
    util, traffic = tmp_path / "util.txt", tmp_path / "gemv.txt"
    monkeypatch.setattr(bench, "UTIL_FILE", str(util))
    monkeypatch.setattr(bench, "GEMV_TRAFFIC_FILE", str(traffic))
    bench.summarize_utilisation(str(run), {"adaln.awq_gemv": 12.5, "mlp_up.gemm_w4a4": 200.0})
    u = dict(l.split(": ", 1) for l in util.read_text().splitlines() if not l.startswith("#"))
    assert u["MfmaUtil_percent"].startswith("35.5")
    assert u["VALUBusy_percent"].startswith("72.0")
    assert u["valu_insts_per_wave_group"].startswith("200.0")
    assert u["mfma_insts_per_wave_group"].startswith("10.00")
    assert u["source_sha256"] == bench.gemm_int4_source_hash()
    assert u["effective_clock_MHz"].startswith("1500")          # 300000 cycles in 200 us
    assert u["cycles_per_wave_group_per_SIMD"].startswith(f"{300000 / (wg / 1024):.0f}")
    t = dict(l.split(": ", 1) for l in traffic.read_text().splitlines() if not l.startswith("#"))
    fetch = 15625.0 * 1024 * 2          # KiB -> bytes, times the copy factor 2
    assert int(t["fetch_bytes_per_launch"]) == int(fetch)
    assert int(t["write_bytes_per_launch"]) == 36 * 1024
    gbps = (fetch + 36 * 1024) / 12.5 / 1e3
    assert t["measured_hbm_GBps"].startswith(f"{gbps:.0f}")
