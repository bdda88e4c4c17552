"""Host logic of bench.py, no GPU: the one-GPU refusal, the FLOP and byte
counts it prices with, and the records it writes from rocprofv3 CSV output
(fed here with synthetic CSVs whose expected figures are worked out by hand)."""

import csv
import os
import subprocess
import sys
import time
import types

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


def _ctr_rows_timed(kernel, counters, dur_ns, dispatches=2, start=0):
    rows, t = [], start
    for i in range(dispatches):
        for name, val in counters.items():
            rows.append({"Dispatch_Id": str(start + i), "Kernel_Name": kernel, "Counter_Name": name,
                         "Counter_Value": str(val), "Start_Timestamp": str(t), "End_Timestamp": str(t + dur_ns)})
        t += dur_ns + 10
    return rows


def test_sq_summary_from_synthetic_run(tmp_path):
    # 2 dispatches of 5 ms at 2.0 GHz: 1e7 cycles per XCD, GRBM_GUI_ACTIVE sums 8 XCDs;
    # MFMA busy on 40 % of 1024 SIMDs' cycles; 1 LDS conflict cycle per 100 active
    cycles = 2.0e9 * 5e-3
    counters = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * cycles * 1024,
                "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 1000.0, "SQ_INSTS_LDS": 3.0e8,
                "SQ_INSTS_MFMA": 5.0e8, "SQ_INSTS_VALU": 2.0e9}
    rows = (_ctr_rows_timed(FWD, counters, 5_000_000)
            + _ctr_rows_timed("other_kernel", {"GRBM_GUI_ACTIVE": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0}, 1000,
                              start=100))
    _write_csv(tmp_path / "ctr.csv", rows)
    ds = bench.read_dispatches(str(tmp_path / "ctr.csv"))
    assert len(ds) == 4
    flops = bench.attention_flops(8, 32, 16384, 128, True)
    rec = bench.sq_summary(ds, "fwd_bf16_kernel", flops)
    assert rec["dispatches"] == 2
    assert rec["engine_clock_ghz"] == pytest.approx(2.0, abs=1e-3)
    assert rec["mfma_busy_frac"] == pytest.approx(0.4, abs=1e-4)
    assert rec["lds_bank_conflict_frac"] == pytest.approx(0.01, abs=1e-4)
    assert rec["clock_adjusted_peak_tflops"] == pytest.approx(256 * 4096 * 2.0e9 / 1e12, abs=0.1)
    assert rec["profiled_duration_ms"] == pytest.approx(5.0, abs=1e-3)
    assert rec["valu_per_mfma"] == pytest.approx(4.0)
    # 5e8 MFMAs of 32768 FLOPs against 4 N^2 d B H / 2 at the headline shape
    assert rec["mfma_flops_over_algorithmic"] == pytest.approx(5.0e8 * 32768 / flops, abs=1e-4)
    assert bench.sq_summary(ds, "bwd_dq_kernel") is None


def test_tcc_summary_scales_by_the_copy_and_checks_decode(tmp_path):
    # the 1 GiB runtime copy reads 0.5 GiB on the read counter (scale 2) and 1 GiB
    # on the write counter (scale 1); a bf16 cast reading more must not be taken for it
    rd, wr = bench.TCC_COUNTERS
    gib32 = (1 << 30) / 32
    rows = (_ctr_rows_timed("__amd_rocclr_copyBuffer", {rd: gib32 / 2, wr: gib32}, 1000, 1)
            + _ctr_rows_timed("void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel",
                              {rd: 2 * gib32, wr: gib32}, 1000, 1, start=10)
            + _ctr_rows_timed(FWD, {rd: 1.0e8, wr: 3.0e7}, 1000, 2, start=20)
            + _ctr_rows_timed("void fa::(anonymous namespace)::decode_kernel<128, 2, 2, true>(...)",
                              {rd: 3.0e7, wr: 1.0}, 1000, 2, start=30))
    _write_csv(tmp_path / "t.csv", rows)
    t = bench.tcc_summary(bench.read_dispatches(str(tmp_path / "t.csv")), 4.0e9, 2.0e9)
    assert t["copy_read_scale"] == pytest.approx(2.0) and t["copy_write_scale"] == pytest.approx(1.0)
    assert t["fwd_read_bytes"] == pytest.approx(32 * 1.0e8 * 2)
    assert t["fwd_write_bytes"] == pytest.approx(32 * 3.0e7)
    assert t["fwd_traffic_over_algorithmic"] == pytest.approx((6.4e9 + 9.6e8) / 4.0e9, abs=1e-4)
    assert t["decode_read_over_known"] == pytest.approx(32 * 3.0e7 * 2 / 2.0e9, abs=1e-4)


def test_kernel_trace_average_skips_warmup(tmp_path):
    _write_csv(tmp_path / "k.csv", _trace_rows(FWD, [9_000_000, 9_000_000, 5_000_000, 7_000_000]))
    ds = bench.read_dispatches(str(tmp_path / "k.csv"))
    ms, n = bench.kernel_avg_ms(ds, "fwd_bf16_kernel", skip=2)
    assert n == 2 and ms == pytest.approx(6.0)


def test_profile_child_commands():
    # the program follows `--` directly (no launcher in between); counter passes
    # stay within one pass's counter budget and never add a system trace
    for kind in ("trace", "sq", "tcc"):
        cmd = bench.child_command(kind, "/tmp/x", "rocprofv3", "python3")
        i = cmd.index("--")
        assert cmd[i + 1] == "python3" and cmd[i + 2].endswith("bench.py") and cmd[i + 3:] == ["--profile-child", kind]
        assert not {"-s", "--sys-trace", "-r", "--runtime-trace", "--hip-trace", "--hsa-trace"} & set(cmd)
        if kind != "trace":
            pmc = cmd[cmd.index("--pmc") + 1:cmd.index("--output-format")]
            assert sum(c.startswith("SQ_") for c in pmc) <= 8 and sum(c.startswith("TCC_") for c in pmc) <= 4
            assert sum(c.startswith("GRBM_") for c in pmc) <= 2
            assert "--kernel-trace" not in cmd


def test_host_cores_respects_affinity_and_omp_cap(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench._host_cores() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench._host_cores() == len(os.sched_getaffinity(0))


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


def test_clock_sampler_reads_the_current_levels(tmp_path):
    # the sysfs files' format: one "index: value unit" line per level, the
    # current one marked with '*'; hwmon power in microwatts
    card = tmp_path / "device"
    (card / "hwmon" / "hwmon3").mkdir(parents=True)
    (card / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1793Mhz *\n2: 2400Mhz\n")
    (card / "pp_dpm_mclk").write_text("0: 900Mhz\n1: 2000Mhz *\n")
    (card / "hwmon" / "hwmon3" / "power1_average").write_text("1360000000\n")
    s = bench.ClockSampler(types.SimpleNamespace(pci_domain_id=-1, pci_bus_id=-1, pci_device_id=-1),
                           period_s=0.001)
    assert s.card is None
    assert "error" in s.summary()
    s.card = str(card)
    s.start()
    time.sleep(0.05)
    s.stop()
    out = s.summary()
    assert out["sclk_mhz"]["median"] == 1793.0 and out["sclk_mhz"]["samples"] >= 1
    assert out["mclk_mhz"]["max"] == 2000.0
    assert out["power_w"]["min"] == 1360.0
