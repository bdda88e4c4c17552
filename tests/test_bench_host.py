"""Host logic of bench.py, no GPU: the one-GPU refusal, the FLOP and byte
counts it prices with, and the records it writes from rocprofv3 CSV output
(fed here with synthetic CSVs whose expected figures are worked out by hand)."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FWD = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, 8, 64, 4, true, false>(...)"


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(kernel, counters, dispatches=2):
    return [{"Dispatch_Id": str(i), "Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": str(val)}
            for i in range(dispatches) for name, val in counters.items()]


def _trace_rows(kernel, durations_ns, start=1000):
    rows, t = [], start
    for d in durations_ns:
        rows.append({"Dispatch_Id": str(len(rows)), "Kernel_Name": kernel,
                     "Start_Timestamp": str(t), "End_Timestamp": str(t + d)})
        t += d + 10
    return rows


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flop_and_byte_counts_of_the_headline_workload():
    # 4 N^2 d B H, halved under the causal mask; Q, K, V read and O written in
    # bf16 plus lse in fp32: 4 * 8*32*16384*128*2 + 8*32*16384*4
    assert bench.attention_flops(8, 32, 16384, 128, True) == 4 * 16384 ** 2 * 128 * 8 * 32 / 2
    assert bench.attention_flops(8, 32, 2048, 128, False) == 4 * 2048 ** 2 * 128 * 8 * 32
    assert bench.algorithmic_fwd_bytes(8, 32, 16384, 128) == 4311744512
    # shared key/value heads: K and V bytes shrink with Hkv, Q, O and lse do not
    assert bench.algorithmic_fwd_bytes(8, 32, 16384, 128, 8) == (2 * 32 + 2 * 8) * 8 * 16384 * 128 * 2 + 4 * 8 * 32 * 16384


def test_counter_record_from_synthetic_run(tmp_path):
    # 2 dispatches of 5 ms at 2.0 GHz: 1e7 cycles per XCD, GRBM_GUI_ACTIVE sums 8 XCDs;
    # MFMA busy on 40 % of 1024 SIMDs' cycles; 1 LDS conflict cycle per 100 active
    cycles = 2.0e9 * 5e-3
    counters = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * cycles * 1024,
                "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 1000.0, "SQ_INSTS_LDS": 3.0e8,
                "SQ_INSTS_MFMA": 5.0e8, "SQ_INSTS_VALU": 2.0e9}
    _write_csv(tmp_path / "ctr.csv", _counter_rows(FWD, counters) + _counter_rows("other_kernel", {
        "GRBM_GUI_ACTIVE": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0}))
    _write_csv(tmp_path / "trace.csv", _trace_rows(FWD, [5_000_000, 5_000_000]))
    out = tmp_path / "rec.md"
    bench.counters_summary(str(tmp_path / "ctr.csv"), str(tmp_path / "trace.csv"), out=str(out))
    rec = bench.read_record(str(out))
    assert float(rec["engine_clock_ghz"]) == pytest.approx(2.0, abs=1e-3)
    assert float(rec["mfma_busy_frac"]) == pytest.approx(0.4, abs=1e-4)
    assert float(rec["lds_bank_conflict_frac"]) == pytest.approx(0.01, abs=1e-4)
    assert float(rec["clock_adjusted_peak_tflops"]) == pytest.approx(256 * 4096 * 2.0e9 / 1e12, abs=0.1)
    assert float(rec["duration_ms"]) == pytest.approx(5.0, abs=1e-3)
    # 5e8 MFMAs of 32768 FLOPs against 4 N^2 d B H / 2 at the headline shape
    assert float(rec["mfma_flops_over_algorithmic"]) == pytest.approx(
        5.0e8 * 32768 / (2 * 16384 ** 2 * 128 * 256), abs=1e-4)


def test_record_of_other_kernel_sources_is_ignored(tmp_path):
    out = tmp_path / "rec.md"
    out.write_text("kernel_source_sha256: " + "0" * 64 + "\nmfma_busy_frac: 0.5\n")
    assert bench.read_record(str(out)) == {}
    out.write_text(f"kernel_source_sha256: {bench.fwd_source_hash()}\nmfma_busy_frac: 0.5\n")
    assert bench.read_record(str(out))["mfma_busy_frac"] == "0.5"
    assert bench.read_record(str(tmp_path / "missing.md")) == {}


def test_traffic_record_scales_by_the_copy(tmp_path):
    # the 1 GiB copy reads 0.5 GiB on FETCH_SIZE (scale 2) and 1 GiB on WRITE_SIZE (scale 1)
    gib_kib = (1 << 30) / 1024.0
    fetch = (_counter_rows("void at::native::copy_kernel<float>", {"FETCH_SIZE": gib_kib / 2}, 1)
             + _counter_rows("void at::native::copy_kernel<float>", {"FETCH_SIZE": 100.0}, 1)
             + _counter_rows(FWD, {"FETCH_SIZE": 1000.0}, 2))
    write = (_counter_rows("void at::native::copy_kernel<float>", {"WRITE_SIZE": gib_kib}, 1)
             + _counter_rows(FWD, {"WRITE_SIZE": 300.0}, 2))
    _write_csv(tmp_path / "f.csv", fetch)
    _write_csv(tmp_path / "w.csv", write)
    out = tmp_path / "traffic.md"
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out=str(out))
    assert bench.read_traffic(str(out)) == pytest.approx(1000.0 * 1024 * 2 + 300.0 * 1024 * 1, abs=1.0)
    out.write_text(out.read_text().replace(bench.fwd_source_hash(), "f" * 64))
    assert bench.read_traffic(str(out)) is None


def test_ceiling_record_picks_the_gemm(tmp_path):
    gemm = "Cijk_Ailk_Bljk_BBS_BH_MT256x256x64"
    dur_ns = 6_000_000
    cycles = 1.7e9 * dur_ns * 1e-9
    ctr = (_counter_rows(gemm, {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.7 * cycles * 1024,
                                "SQ_BUSY_CU_CYCLES": 1.0}, 3)
           + _counter_rows("elementwise_kernel", {"GRBM_GUI_ACTIVE": 5.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.0,
                                                  "SQ_BUSY_CU_CYCLES": 1.0}, 3))
    trace = _trace_rows(gemm, [dur_ns] * 3) + _trace_rows("elementwise_kernel", [50_000] * 3, start=10 ** 9)
    _write_csv(tmp_path / "c.csv", ctr)
    _write_csv(tmp_path / "t.csv", trace)
    out = tmp_path / "ceil.md"
    bench.ceiling_summary(str(tmp_path / "c.csv"), str(tmp_path / "t.csv"), out=str(out))
    rec = bench.read_ceiling(str(out))
    assert rec["kernel"].startswith("Cijk")
    assert float(rec["tflops"]) == pytest.approx(2 * 16384 ** 3 / 6e-3 / 1e12, rel=1e-3)
    assert float(rec["engine_clock_ghz"]) == pytest.approx(1.7, abs=1e-3)
    assert float(rec["mfma_busy_frac"]) == pytest.approx(0.7, abs=1e-4)
