"""Benchmark of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-profile]
                    [--profile-out DIR] [--workload NAME]

Workload: the causal bf16 forward at B=8, H=32, N=16384, d=128 (the "16K
tokens x 32 heads x batch 8" shape of "FlashAttention" (tensorlab.fun), Beat
01), inputs i.i.d. N(0, 1) from a fixed seed, resident in HBM before timing.
A step is one fa_forward call over the whole batch; `value` is attention
TFLOP/s = 4 N^2 d B H (halved for causal) / step time.

Prints exactly one JSON line on stdout (progress goes to stderr). Besides the
headline it carries, each timed in the same process:
  fwd_bwd      fa_forward + fa_backward at the headline shape (3.5x the FLOPs);
  configs      the other configured shapes: non-causal B8 H32 N2048 (Q x4),
               cold- and warm-cache; causal B1 H8 N100000; the backward of
               causal B4 H16 N4096;
  worst_case   the forward on rising-score inputs, where the fast pass's
               row-sum bound fails in every query block;
  widened      decode (100K- and 16K-token caches), the fp8 forward, the
               block-sparse forward and 8 shared key/value heads, each timed
               as its own --workload line would, with fewer steps;
  ceiling      the vendor bf16 GEMM at 16384^3 (what a plain matrix product
               reaches on this part);
  roofline     the forward against the dense-bf16 matrix peak (2516.6 TFLOP/s
               = 256 CUs x 4096 FLOP/clk x 2.4 GHz), per-launch durations from
               HIP events on the launch stream, and its HBM traffic;
  profile      rocprofv3 runs of this same script, started as child processes
               before this process touches the GPU: the kernel-trace average
               of each kernel (to set beside the HIP-event figures), SQ
               counters (matrix-core busy, engine clock, LDS bank conflicts,
               instruction mix) and the DRAM-side byte counters
               (TCC_EA0_RDREQ_DRAM_32B, TCC_EA0_WRREQ_WRITE_DRAM_32B, in
               32-byte units), scaled by their reading for a 1 GiB device copy
               and checked on the decode kernel, whose K/V bytes are known;
  clocks       engine and memory clock (and board power where the driver
               exposes it) sampled from the card's sysfs files while the
               headline's timed launches run;
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload.
"""

import argparse
import json
import os
import shutil
import subprocess
import sys
import tempfile
import time


def _host_cores():
    """Cores the CPU oracle may use: this process's CPU affinity, capped by an
    OMP_NUM_THREADS the environment already sets (a share of a larger host)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


# (before numpy is imported by anything: its BLAS reads these once)
HOST_CORES = _host_cores()
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(HOST_CORES))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd (and fwd+bwd) at N=16K d=128 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU * 4096 FLOP/clk/CU * 2.4 GHz, dense bf16
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 matrix peak, twice the bf16 one
N_XCD, N_CU, SIMD_PER_CU, FLOP_PER_CLK_CU = 8, 256, 4, 4096
MFMA_FLOPS = 32 * 32 * 16 * 2  # one v_mfma_f32_32x32x16_bf16
GEMM_N = 16384
COPY_BYTES = 1 << 30
CEILING_FILE = os.path.join(ROOT, "profiles", "gemm_bf16_ceiling_m16384n16384k16384.md")
CEILING_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
# one --pmc pass each (at most 8 SQ, 4 TCC and 2 GRBM counters per pass)
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
               "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"]
TCC_COUNTERS = ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]
CHILD_TIMEOUT_S = 240
# minimum warm-up wall time before timing the shorter workloads (the headline
# keeps exactly --warmup steps)
WARM_MS = 150.0
# kernels named in the records (substring of the demangled name -> short name)
KERNELS = {"fwd_bf16_kernel": "fwd_bf16_kernel", "bwd_dkdv_kernel": "bwd_dkdv_kernel",
           "bwd_dq_kernel": "bwd_dq_kernel", "bwd_preprocess_kernel": "bwd_preprocess_kernel",
           "decode_kernel": "decode_kernel", "merge_kernel": "merge_kernel", "merge_wide_kernel": "merge_wide_kernel",
           "fwd_fp8_kernel": "fwd_fp8_kernel", "fwd_f32_kernel": "fwd_f32_kernel"}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def attention_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def algorithmic_fwd_bytes(B, H, N, d, Hkv=None):
    """Q, K, V read once and O written once (bf16), lse written once (fp32)."""
    Hkv = H if Hkv is None else Hkv
    return (2.0 * H + 2.0 * Hkv) * B * N * d * 2 + 4.0 * B * H * N


def decode_bytes(cfg):
    """Algorithmic bytes of one decode call: K and V read once, Q read, O and lse written."""
    B, H, Hkv, Nq, Nk, d = (cfg[x] for x in ("B", "H", "Hkv", "Nq", "Nk", "d"))
    return 2.0 * B * Hkv * Nk * d * 2 + 2.0 * B * H * Nq * d * 2 + 4.0 * B * H * Nq


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload configuration id (3 = headline)")
    ap.add_argument("--workload", choices=["gqa", "mqa", "decode", "decode_gqa", "decode_long", "sparse", "fp8",
                                           "rising", "gemm_ceiling"],
                    help="instead of --config: the same causal 16K shape with 8 (gqa) or 1 (mqa) "
                         "key/value heads shared by the 32 query heads, or a decode workload (one "
                         "query per head against a 16K or 100K-token cache), or the block-sparse "
                         "forward on the causal 16K shape (first block + diagonal + 1/8 of the rest), "
                         "or the fp8 (e4m3) forward on the causal 16K shape, or the forward on "
                         "rising-score inputs, or (context, not the library) the vendor bf16 GEMM "
                         "torch.matmul at 16384^3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the fwd+bwd timing")
    ap.add_argument("--no-extra", action="store_true", help="skip the other configurations and the worst case")
    ap.add_argument("--no-profile", action="store_true", help="skip the rocprofv3 child runs")
    ap.add_argument("--profile-out", metavar="DIR",
                    help="keep the rocprofv3 output and write the summary records into DIR")
    ap.add_argument("--profile-child", choices=["trace", "sq", "tcc"], help=argparse.SUPPRESS)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "WORKLOAD"),
                    help="no GPU work: turn the run_kernel_stats.csv of one rocprofv3 --kernel-trace --stats run "
                         "of `bench.py --workload WORKLOAD` into a kernel-statistics record (stdout)")
    ap.add_argument("--ceiling-summary", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                    help="no GPU work: turn one rocprofv3 --pmc --kernel-trace run of "
                         "`bench.py --workload gemm_ceiling` into the GEMM ceiling record under profiles/")
    return ap.parse_args(argv)


# ---------------------------------------------------------------- rocprofv3 output


def short_name(name):
    for key, short in KERNELS.items():
        if key in name:
            return short
    if "copyBuffer" in name:  # the runtime's device-to-device copy (torch's same-dtype copy_)
        return "device_copy"
    name = name[5:] if name.startswith("void ") else name
    return name.replace("(anonymous namespace)::", "").split("(")[0][:60]


def read_dispatches(path):
    """One dict per dispatch from a rocprofv3 csv (kernel trace or counter
    collection): name, duration (ns) and {counter: value}."""
    import csv

    out = {}
    for r in csv.DictReader(open(path)):
        key = r.get("Dispatch_Id") or str(len(out))
        d = out.get(key)
        if d is None:
            d = out[key] = {"name": r["Kernel_Name"], "short": short_name(r["Kernel_Name"]), "counters": {},
                            "dur_ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                            if r.get("End_Timestamp") else None}
        if "Counter_Name" in r and r["Counter_Name"]:
            d["counters"][r["Counter_Name"]] = d["counters"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return list(out.values())


def kernel_avg_ms(dispatches, short, skip=0):
    durs = [d["dur_ns"] for d in dispatches if d["short"] == short][skip:]
    return (sum(durs) / len(durs) * 1e-6, len(durs)) if durs else (None, 0)


def sq_summary(dispatches, short, algorithmic_flops=None):
    """Matrix-core busy fraction, engine clock and the rest of the SQ pass for
    one kernel, averaged over its dispatches. GRBM_GUI_ACTIVE sums the 8 XCDs:
    clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 256 CU x 4 SIMD)."""
    ds = [d for d in dispatches if d["short"] == short and "GRBM_GUI_ACTIVE" in d["counters"]]
    if not ds:
        return None
    mean = lambda k: sum(d["counters"].get(k, 0.0) for d in ds) / len(ds)
    dur = sum(d["dur_ns"] for d in ds) / len(ds) * 1e-9
    cycles = mean("GRBM_GUI_ACTIVE") / N_XCD
    clock = cycles / dur / 1e9
    out = {
        "dispatches": len(ds),
        "profiled_duration_ms": round(dur * 1e3, 4),
        "engine_clock_ghz": round(clock, 3),
        "clock_adjusted_peak_tflops": round(N_CU * FLOP_PER_CLK_CU * clock * 1e9 / 1e12, 1),
        "mfma_busy_frac": round(mean("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * N_CU * SIMD_PER_CU), 4),
        "lds_bank_conflict_frac": round(mean("SQ_LDS_BANK_CONFLICT") / max(mean("SQ_LDS_IDX_ACTIVE"), 1.0), 4),
        "mfma_instructions": mean("SQ_INSTS_MFMA"),
        "valu_per_mfma": round(mean("SQ_INSTS_VALU") / max(mean("SQ_INSTS_MFMA"), 1.0), 3),
        "lds_per_mfma": round(mean("SQ_INSTS_LDS") / max(mean("SQ_INSTS_MFMA"), 1.0), 3),
    }
    if algorithmic_flops:
        out["mfma_flops_over_algorithmic"] = round(mean("SQ_INSTS_MFMA") * MFMA_FLOPS / algorithmic_flops, 4)
    return out


def tcc_summary(dispatches, fwd_algorithmic_bytes, decode_known_bytes):
    """DRAM-side bytes (32-byte units of TCC_EA0_RDREQ_DRAM_32B / WRREQ_WRITE_DRAM_32B)
    of the forward, scaled per direction by what the counters read for the
    COPY_BYTES device copy (the largest runtime copy in the pass), and the decode
    kernel's read bytes against the K/V bytes it must read exactly once."""
    rd, wr = TCC_COUNTERS
    copies = [d for d in dispatches if d["short"] == "device_copy" and rd in d["counters"]]
    if not copies:
        return None
    copy = max(copies, key=lambda d: d["counters"][rd])
    rd_scale = COPY_BYTES / max(32.0 * copy["counters"][rd], 1.0)
    wr_scale = COPY_BYTES / max(32.0 * copy["counters"].get(wr, 0.0), 1.0)
    per = lambda short, key, scale: [32.0 * d["counters"][key] * scale for d in dispatches
                                     if d["short"] == short and key in d["counters"]]
    f_rd, f_wr = per("fwd_bf16_kernel", rd, rd_scale), per("fwd_bf16_kernel", wr, wr_scale)
    dec_rd = per("decode_kernel", rd, rd_scale)
    if not f_rd or not f_wr:
        return None
    fwd_read, fwd_write = sum(f_rd) / len(f_rd), sum(f_wr) / len(f_wr)
    out = {
        "copy_read_scale": round(rd_scale, 4),
        "copy_write_scale": round(wr_scale, 4),
        "fwd_read_bytes": fwd_read,
        "fwd_write_bytes": fwd_write,
        "fwd_traffic_bytes": fwd_read + fwd_write,
        "fwd_algorithmic_bytes": fwd_algorithmic_bytes,
        "fwd_traffic_over_algorithmic": round((fwd_read + fwd_write) / fwd_algorithmic_bytes, 4),
        "fwd_dispatches": len(f_rd),
    }
    if dec_rd:
        out["decode_read_bytes"] = sum(dec_rd) / len(dec_rd)
        out["decode_known_bytes"] = decode_known_bytes
        out["decode_read_over_known"] = round(out["decode_read_bytes"] / decode_known_bytes, 4)
    return out


# ---------------------------------------------------------------- rocprofv3 child runs


def rocprof_bin():
    for cand in (shutil.which("rocprofv3"), "/opt/rocm/bin/rocprofv3"):
        if cand and os.path.exists(cand):
            return cand
    return None


def child_command(kind, outdir, rocprof="rocprofv3", python=None):
    """The rocprofv3 command of one child pass (the program follows `--` directly)."""
    python = python or sys.executable
    prog = ["--", python, os.path.join(ROOT, "bench.py"), "--profile-child", kind]
    common = ["--output-format", "csv", "-d", os.path.join(outdir, kind), "-o", "run"]
    if kind == "trace":
        return [rocprof, "--kernel-trace", "--stats", *common, *prog]
    counters = SQ_COUNTERS if kind == "sq" else TCC_COUNTERS
    return [rocprof, "--pmc", *counters, *common, *prog]


def profile_child(a):
    """GPU work of one child pass (run under rocprofv3 by the parent)."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.config(3)
    B, H, N, d, causal, scale = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"], cfg["scale"]
    if a.profile_child == "tcc":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    q, k, v, do = W.make_inputs(cfg, dev, with_do=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    fwd = lambda: fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    n_fwd = {"trace": 12, "sq": 2, "tcc": 2}[a.profile_child]
    for _ in range(n_fwd):
        fwd()
    torch.cuda.synchronize()
    if a.profile_child in ("trace", "sq"):
        ws = torch.empty(fa.backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        for _ in range(3 if a.profile_child == "trace" else 1):
            fwd()
            fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, workspace=ws)
        torch.cuda.synchronize()
    if a.profile_child == "tcc":
        del q, k, v, do, o
        dcfg = W.DECODE_WORKLOADS["decode"]
        dq_, dk_, dv_ = W.make_decode_inputs(dcfg, dev)
        for _ in range(2):
            fa.decode(dq_, dk_, dv_, causal=dcfg["causal"])
        torch.cuda.synchronize()
    # (in the pass's output directory: tells the parent the program completed)
    outdir = os.environ.get("BENCH_CHILD_DIR")
    if outdir:
        open(os.path.join(outdir, "child_done"), "w").close()


def headline_profile(paths, errors, launch_avg_ms):
    """Parse the three passes ({kind: csv path or None}) into the JSON line's
    profile block."""
    errors = list(errors)
    cfg3 = dict(B=8, H=32, N=16384, d=128)
    fwd_flops = attention_flops(8, 32, 16384, 128, True)
    prof = {"source": "rocprofv3 child runs of this bench.py invocation on the same GPU, before its timed region "
                      "(profiled launches)", "errors": errors}
    if paths.get("trace"):
        ds = read_dispatches(paths["trace"])
        fwd_ms, n = kernel_avg_ms(ds, "fwd_bf16_kernel", skip=2)
        prof["kernel_trace"] = {"fwd_bf16_kernel_avg_ms": round(fwd_ms, 4) if fwd_ms else None,
                                "fwd_launches": n}
        for kname in ("bwd_preprocess_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
            ms, n = kernel_avg_ms(ds, kname)
            prof["kernel_trace"][f"{kname}_avg_ms"] = round(ms, 4) if ms else None
        if fwd_ms:
            prof["kernel_trace"]["fwd_over_hip_event_launch_avg"] = round(fwd_ms / launch_avg_ms, 4)
            prof["kernel_trace"]["fwd_frac_of_peak"] = round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    if paths.get("sq"):
        ds = read_dispatches(paths["sq"])
        bwd_products = {"bwd_dkdv_kernel": 4, "bwd_dq_kernel": 3}
        prof["counters"] = {
            "fwd_bf16_kernel": sq_summary(ds, "fwd_bf16_kernel", fwd_flops),
            "bwd_dkdv_kernel": sq_summary(ds, "bwd_dkdv_kernel", fwd_flops / 2 * bwd_products["bwd_dkdv_kernel"]),
            "bwd_dq_kernel": sq_summary(ds, "bwd_dq_kernel", fwd_flops / 2 * bwd_products["bwd_dq_kernel"]),
        }
        f = prof["counters"]["fwd_bf16_kernel"]
        if f:
            f["frac_of_clock_adjusted_peak"] = round(
                fwd_flops / (launch_avg_ms * 1e-3) / 1e12 / f["clock_adjusted_peak_tflops"], 4)
    if paths.get("tcc"):
        dcfg = dict(B=8, H=32, Hkv=32, Nq=1, Nk=16384, d=128)
        known = 2.0 * dcfg["B"] * dcfg["Hkv"] * dcfg["Nk"] * dcfg["d"] * 2
        prof["traffic"] = tcc_summary(read_dispatches(paths["tcc"]), algorithmic_fwd_bytes(**cfg3), known)
    return prof


def write_profile_records(outdir, paths, prof, launch_avg_ms):
    """Text records of the three passes (for profiles/)."""
    import csv

    cmd_parent = "python bench.py --profile-out <out>"
    lines_cmd = lambda kind: "  " + " ".join(child_command(kind, "<out>", "rocprofv3", "python3")).replace(
        os.path.join(ROOT, "bench.py"), "bench.py")
    if paths.get("trace"):
        stats = os.path.join(os.path.dirname(paths["trace"]), "run_kernel_stats.csv")
        rows = list(csv.DictReader(open(stats))) if os.path.exists(stats) else []
        kt = prof.get("kernel_trace", {})
        out = [
            "Kernel statistics (rocprofv3 --kernel-trace --stats) of the causal bf16 attention forward and backward,",
            "B=8 H=32 N=16384 d=128, one MI355X: 12 forward launches (the first 2 are warm-up), then 3 fwd+bwd steps.",
            f"Made by `{cmd_parent}` (from the repository root), which runs, before its own timed region:",
            lines_cmd("trace"),
            "",
            f"{'kernel':62s} {'calls':>6s} {'average_ns':>12s} {'min_ns':>12s} {'max_ns':>12s}",
        ]
        for r in rows:
            out.append(f"{short_name(r['Name'])[:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']):12.0f} "
                       f"{float(r['MinNs']):12.0f} {float(r['MaxNs']):12.0f}")
        fwd_flops = attention_flops(8, 32, 16384, 128, True)
        if kt.get("fwd_bf16_kernel_avg_ms"):
            fm = kt["fwd_bf16_kernel_avg_ms"]
            out += ["",
                    f"fwd_bf16_kernel, launches 3-12: {fm:.4f} ms = {fwd_flops / (fm * 1e-3) / 1e12:.1f} TFLOP/s "
                    f"({fwd_flops / (fm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS:.4f} of the 2516.6 dense-bf16 peak)",
                    f"the same invocation's unprofiled HIP-event launch average: {launch_avg_ms:.4f} ms "
                    f"(ratio {fm / launch_avg_ms:.4f})"]
        dk, dq = kt.get("bwd_dkdv_kernel_avg_ms"), kt.get("bwd_dq_kernel_avg_ms")
        pre = kt.get("bwd_preprocess_kernel_avg_ms")
        if dk and dq and pre:
            bwd = dk + dq + pre
            out += [f"backward kernels {pre:.3f} + {dk:.3f} + {dq:.3f} = {bwd:.3f} ms: "
                    f"{2.5 * fwd_flops / (bwd * 1e-3) / 1e12:.1f} TFLOP/s at the 5-product count "
                    f"({2.5 * fwd_flops / (bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS:.4f} of peak)"]
        open(os.path.join(outdir, "fwd_bwd_kernels_causal_b8h32n16384d128.txt"), "w").write("\n".join(out) + "\n")
    if prof.get("counters"):
        out = ["# SQ counters of the causal bf16 attention kernels, B=8 H=32 N=16384 d=128, one MI355X",
               f"# Made by `{cmd_parent}` (from the repository root), which runs before its timed region:",
               "# " + lines_cmd("sq").strip(),
               "# engine clock = GRBM_GUI_ACTIVE / 8 XCDs / profiled kernel duration;",
               "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 256 CU x 4 SIMD);",
               "# mfma_flops_over_algorithmic: 32768 FLOPs per v_mfma_f32_32x32x16_bf16 against the kernel's",
               "# algorithmic count (forward 2 N^2 d per causal head; dK/dV 4 and dQ 3 products)."]
        for kname, rec in prof["counters"].items():
            if rec:
                out.append(f"{kname}: " + json.dumps(rec))
        open(os.path.join(outdir, "fwd_bwd_counters_causal_b8h32n16384d128.md"), "w").write("\n".join(out) + "\n")
    if prof.get("traffic"):
        t = prof["traffic"]
        out = ["# DRAM-side traffic of fwd_bf16_kernel, causal bf16 attention forward B=8 H=32 N=16384 d=128,",
               "# one MI355X. Bytes = 32 x TCC_EA0_RDREQ_DRAM_32B (reads) and 32 x TCC_EA0_WRREQ_WRITE_DRAM_32B",
               "# (writes), summed over the L2 channels: requests the L2 sends toward memory (the memory-side",
               "# Infinity Cache may serve some reads), each direction scaled by its reading for a plain",
               "# 1 GiB torch copy in the same pass. Check: the decode kernel reads each K/V byte once.",
               f"# Made by `{cmd_parent}` (from the repository root), which runs before its timed region:",
               "# " + lines_cmd("tcc").strip()]
        for key, val in t.items():
            out.append(f"{key}: {val}")
        open(os.path.join(outdir, "fwd_bf16_traffic_causal_b8h32n16384d128.md"), "w").write("\n".join(out) + "\n")


# ---------------------------------------------------------------- timing


class ClockSampler:
    """Engine and memory clock (and board power, where the driver exposes it)
    read from the amdgpu sysfs files of this GPU's card every `period_s` on a
    host thread while the timed launches run: pp_dpm_sclk / pp_dpm_mclk mark
    the current level with '*'; hwmon power1_average / power1_input are in
    microwatts. Plain file reads, no child process; silent if the files are
    not there."""

    def __init__(self, props, period_s=0.02):
        import threading
        self.period_s = period_s
        self.card = self._card_dir(props)
        self.samples = {"sclk_mhz": [], "mclk_mhz": [], "power_w": []}
        self._stop = threading.Event()
        self._thread = None

    @staticmethod
    def _card_dir(props):
        want = (getattr(props, "pci_domain_id", None), getattr(props, "pci_bus_id", None),
                getattr(props, "pci_device_id", None))
        try:
            names = sorted(n for n in os.listdir("/sys/class/drm") if n.startswith("card") and "-" not in n)
        except OSError:
            return None
        for n in names:
            dev = os.path.join("/sys/class/drm", n, "device")
            try:
                dom, bus, rest = os.path.basename(os.path.realpath(dev)).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    return dev
            except (OSError, ValueError):
                continue
        return None

    @staticmethod
    def _current_level(path):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            pass
        return None

    def _power(self):
        import glob
        for name in ("power1_average", "power1_input"):
            for f in glob.glob(os.path.join(self.card, "hwmon", "hwmon*", name)):
                try:
                    return int(open(f).read()) / 1e6
                except (OSError, ValueError):
                    pass
        return None

    def _read(self):
        for key, f in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
            x = self._current_level(os.path.join(self.card, f))
            if x is not None:
                self.samples[key].append(x)
        w = self._power()
        if w is not None:
            self.samples["power_w"].append(w)

    def _run(self):
        while not self._stop.is_set():
            self._read()
            self._stop.wait(self.period_s)

    def start(self):
        import threading
        if self.card is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if self.card is None:
            return {"error": "no amdgpu sysfs card matches this GPU's PCI address"}
        out = {"source": f"amdgpu sysfs {os.path.basename(os.path.realpath(self.card))} (pp_dpm_sclk, "
                         f"pp_dpm_mclk, hwmon power), sampled every {self.period_s * 1e3:.0f} ms on a host "
                         f"thread during the timed launches"}
        for key, xs in self.samples.items():
            if xs:
                s = sorted(xs)
                out[key] = {"median": s[len(s) // 2], "min": s[0], "max": s[-1], "samples": len(s)}
        return out


def time_launches(fn, steps, warmup, stream, between=None, warm_ms=0.0, sampler=None, per_launch=True):
    """Run fn `warmup` times (and, with warm_ms, on until that much wall time
    has passed: a sub-millisecond kernel needs ~0.1 s of work before the
    clocks settle), then `steps` timed times, each bracketed by HIP events on
    `stream`; `between` (untimed) runs before each timed launch; a
    ClockSampler runs from the first timed launch to the end of the last.
    With per_launch=False only one event pair brackets the `steps`
    back-to-back calls (each event record costs the stream ~5 us, which a
    call of well under a millisecond would carry) and every entry of the
    per-launch list is their mean. Returns (ms of the whole timed region,
    per-launch ms list)."""
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(5):
            if between is not None:
                between()
            fn()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if sampler is not None:
        sampler.start()
    if not per_launch:
        assert between is None, "back-to-back timing has no untimed work between calls"
        t_start.record(stream)
        for _ in range(steps):
            fn()
        t_end.record(stream)
        torch.cuda.synchronize()
        if sampler is not None:
            sampler.stop()
        total = t_start.elapsed_time(t_end)
        return total, [total / steps] * steps
    t_start.record(stream)
    for a, b in ev:
        if between is not None:
            between()
        a.record(stream)
        fn()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    if sampler is not None:
        sampler.stop()
    return t_start.elapsed_time(t_end), [a.elapsed_time(b) for a, b in ev]


def _median(xs):
    s = sorted(xs)
    return s[len(s) // 2]


def time_vendor_gemm(steps, warmup):
    """The vendor's bf16 GEMM (torch.matmul -> hipBLASLt) at 16384^3 on the same
    part: what a dense matrix product reaches here under the same power and
    clock limits. Context for the attention kernels' roofline, not a library
    path. Returns (ms per product, TFLOP/s)."""
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    x = torch.randn(GEMM_N, GEMM_N, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    y = torch.randn(GEMM_N, GEMM_N, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    z = torch.empty(GEMM_N, GEMM_N, device=dev, dtype=torch.bfloat16)
    total_ms, _ = time_launches(lambda: torch.matmul(x, y, out=z), steps, warmup, stream)
    ms = total_ms / steps
    del x, y, z
    return ms, 2.0 * GEMM_N ** 3 / (ms * 1e-3) / 1e12


def bench_gemm_ceiling(a):
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms, tflops = time_vendor_gemm(a.steps, a.warmup)
    return {"metric": "vendor bf16 GEMM throughput (context)", "value": round(tflops, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"torch.matmul bf16 {GEMM_N}x{GEMM_N}x{GEMM_N}",
                       "device": torch.cuda.get_device_name(dev)},
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def ceiling_summary(counter_csv, trace_csv, out=None):
    """Write the GEMM ceiling record from one --pmc --kernel-trace run of
    `bench.py --workload gemm_ceiling`: the GEMM kernel is the one with the
    most launches of GEMM_N^3 work (the longest total time in the trace)."""
    import csv

    durs = {}
    for r in csv.DictReader(open(trace_csv)):
        durs.setdefault(r["Kernel_Name"], []).append(
            (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
    name = max(durs, key=lambda k: sum(durs[k]))
    vals = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Kernel_Name"] == name:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = lambda k: sum(vals[k]) / len(vals[k])
    dur = sum(durs[name]) / len(durs[name])
    cycles = mean("GRBM_GUI_ACTIVE") / N_XCD
    sclk = cycles / dur / 1e9
    mfma = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * N_CU * SIMD_PER_CU)
    tflops = 2.0 * GEMM_N ** 3 / dur / 1e12
    lines = [
        f"# Vendor bf16 GEMM (torch.matmul -> hipBLASLt), {GEMM_N}x{GEMM_N}x{GEMM_N}, one MI355X: the ceiling a",
        "# dense matrix product reaches on this part under its power and clock limits.",
        "# Command (from the repository root, cd /tmp && export TMPDIR=/tmp first):",
        "#   rocprofv3 --pmc " + " ".join(CEILING_COUNTERS) + " --kernel-trace --output-format csv -d <out>/gemm -o run \\",
        "#       -- python3 <repo>/bench.py --workload gemm_ceiling --steps 5 --warmup 2",
        "#   python bench.py --ceiling-summary <out>/gemm/run_counter_collection.csv <out>/gemm/run_kernel_trace.csv",
        "# engine clock = GRBM_GUI_ACTIVE / 8 XCDs / kernel duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
        "# (clock cycles x 256 CU x 4 SIMD). Profiled launches, so the duration is the profiler's.",
        f"kernel: {name[:120]}",
        f"launches: {len(durs[name])}",
        f"duration_ms: {dur * 1e3:.3f}",
        f"tflops: {tflops:.1f}",
        f"frac_of_peak: {tflops / PEAK_BF16_TFLOPS:.4f}",
        f"engine_clock_ghz: {sclk:.3f}",
        f"mfma_busy_frac: {mfma:.4f}",
    ]
    with open(out or CEILING_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def workload_figures(workload):
    """(kernel short name, description, algorithmic FLOPs or None, algorithmic bytes or None)
    of one launch of a bench workload's main kernel."""
    from exact_tiled_attention_38_amd import workloads as W

    if workload.startswith("decode"):
        c = W.DECODE_WORKLOADS[workload]
        return ("decode_kernel", f"decode, B={c['B']} H={c['H']} Hkv={c['Hkv']} Nq={c['Nq']} Nk={c['Nk']} "
                f"d={c['d']}; the whole call adds a merge kernel", None, decode_bytes(c))
    if workload == "sparse":
        c = W.SPARSE_WORKLOADS["sparse"]
        rp, cols = W.sparse_selection(c["B"], c["H"], c["N"], c["seed"], c["keep"])
        pairs = W.sparse_visible_pairs(c["N"], rp, cols, c["B"] * c["H"], c["causal"])
        return ("fwd_bf16_kernel", f"block-sparse forward, causal B={c['B']} H={c['H']} N={c['N']} d={c['d']}, "
                f"{cols.shape[0]} listed 256x64 blocks, {pairs:.4g} kept pairs", 4.0 * c["d"] * pairs, None)
    if workload == "fp8":
        c = W.FP8_WORKLOADS["fp8"]
        return ("fwd_fp8_kernel", f"fp8 (e4m3) forward, causal B={c['B']} H={c['H']} N={c['N']} d={c['d']}",
                attention_flops(c["B"], c["H"], c["N"], c["d"], True), None)
    if workload in ("gqa", "mqa"):
        c = W.GQA_WORKLOADS[workload]
        return ("fwd_bf16_kernel", f"forward with shared heads, causal B={c['B']} H={c['H']} Hkv={c['Hkv']} "
                f"N={c['N']} d={c['d']}", attention_flops(c["B"], c["H"], c["N"], c["d"], True),
                algorithmic_fwd_bytes(c["B"], c["H"], c["N"], c["d"], c["Hkv"]))
    raise ValueError(workload)


def stats_summary(stats_csv, workload):
    """Kernel-statistics record of one rocprofv3 --kernel-trace --stats run of
    `bench.py --workload WORKLOAD` (returned as text)."""
    import csv

    kernel, desc, flops, nbytes = workload_figures(workload)
    fp8 = workload == "fp8"
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"Kernel statistics (rocprofv3 --kernel-trace --stats) of bench.py's {workload} workload on one MI355X:",
           desc + ".",
           "Commands (from the repository root, after cd /tmp && export TMPDIR=/tmp):",
           f"  rocprofv3 --kernel-trace --stats --output-format csv -d <out>/{workload} -o run -- \\",
           f"      python3 bench.py --workload {workload} --steps 10 --warmup 2 --no-cpu-baseline",
           f"  python bench.py --stats-summary <out>/{workload}/run_kernel_stats.csv {workload}",
           "",
           f"{'kernel':62s} {'calls':>6s} {'average_ns':>12s} {'min_ns':>12s} {'max_ns':>12s}"]
    avg = None
    for r in rows:
        name = short_name(r["Name"])
        if name == kernel and avg is None:
            avg = float(r["AverageNs"]) * 1e-9
        out.append(f"{name[:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']):12.0f} "
                   f"{float(r['MinNs']):12.0f} {float(r['MaxNs']):12.0f}")
    out.append("")
    if avg and flops:
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        tf = flops / avg / 1e12
        out.append(f"{kernel}: {flops:.4g} algorithmic FLOPs / {avg * 1e3:.4f} ms = {tf:.1f} TFLOP/s "
                   f"({tf / peak:.4f} of the {peak} {'fp8' if fp8 else 'bf16'} peak)")
    if avg and nbytes:
        out.append(f"{kernel}: {nbytes:.4g} algorithmic bytes / {avg * 1e3:.4f} ms = {nbytes / avg / 1e9:.1f} GB/s "
                   f"({nbytes / avg / 1e9 / PEAK_HBM_GBS:.4f} of 8 TB/s)")
    return "\n".join(out) + "\n"


def read_ceiling(path=None):
    try:
        rec = {}
        for line in open(path or CEILING_FILE):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
        return rec if "tflops" in rec else {}
    except OSError:
        return {}


# ---------------------------------------------------------------- the CPU oracle


def cpu_baseline(cfg, q, k, v, target_s):
    """Time the fp64 oracle on whole rows of the same workload until ~target_s of work."""
    import numpy as np

    import oracle
    from exact_tiled_attention_38_amd import workloads as W

    blas_threads = None
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    B, H, N, d, causal, scale = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"], cfg["scale"]
    group = H // cfg.get("Hkv", H)
    heads = W.sample_heads(B, H, B * H, cfg["seed"] + 2)
    rows = W.sample_rows(N, 1024, cfg["seed"] + 1)
    flops, elapsed, done = 0.0, 0.0, 0
    for b, h in heads:
        qh = q[b, h].float().cpu().numpy()
        kh = k[b, h // group].float().cpu().numpy()
        vh = v[b, h // group].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.forward(qh, kh, vh, scale, causal, rows=rows)
        elapsed += time.perf_counter() - t0
        visible = (rows + 1) if causal else np.full_like(rows, N)
        flops += 4.0 * d * float(visible.sum())
        done += 1
        if elapsed >= target_s:
            break
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rate = flops / elapsed
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": HOST_CORES,
        "blas_threads": blas_threads,
        "cpu_model": cpu_model,
        "extrapolated_full_workload_seconds": round(attention_flops(B, H, N, d, causal) / rate, 1),
        "kind": "oracle",
        "sample": f"fp64 one-shot oracle on {len(rows)} seeded rows (full score rows) of each of {done} heads "
                  f"of the same workload; rate = algorithmic attention FLOPs of those rows "
                  f"(4 d x visible keys) / {elapsed:.1f} s; cores = the process's CPU affinity capped by "
                  f"OMP_NUM_THREADS, set for the BLAS before numpy loads",
        "seconds": elapsed,
    }


# ---------------------------------------------------------------- other workloads


def bench_decode(a, cfg):
    """One decode call (split kernel + merge kernel) per step; HBM roofline."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    q, k, v = W.make_decode_inputs(cfg, dev)
    B, H, Hkv, Nq, Nk, d = (cfg[x] for x in ("B", "H", "Hkv", "Nq", "Nk", "d"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device=dev)
    scale = 1.0 / d ** 0.5
    step = lambda: fa.decode(q, k, v, causal=cfg["causal"], scale=scale, workspace=ws, out=o, lse=lse)
    # eager calls back to back under one event pair: a call is 0.07-0.3 ms,
    # and an event pair around each would add ~5 us of stream time to each
    total_ms, per = time_launches(step, a.steps, a.warmup, stream, warm_ms=WARM_MS, per_launch=False)
    ms = total_ms / a.steps
    nbytes = decode_bytes(cfg)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # Serving loops replay captured HIP graphs: time CALLS calls captured in
    # one graph (the same kernels and arguments), which leaves out the gaps
    # between eagerly issued kernels.
    calls = 10
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            step()
    replay_total, _ = time_launches(graph.replay, max(2, a.steps // 2), 2, stream, warm_ms=WARM_MS)
    launch_avg = replay_total / max(2, a.steps // 2) / calls
    achieved = nbytes / (launch_avg * 1e-3) / 1e9
    return {
        "metric": "attention decode: algorithmic HBM bytes per second (K and V read once)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"bf16 decode, B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d}"
                               + (" causal" if cfg["causal"] else ""),
                   "B": B, "H": H, "Hkv": Hkv, "Nq": Nq, "Nk": Nk, "d": d, "causal": bool(cfg["causal"])},
        "eager_ms_per_call": round(ms, 5),
        "graph_ms_per_call": round(launch_avg, 5),
        "roofline": {
            "kernel": "decode_kernel + merge_kernel (one fa_decode call, from HIP-graph replays of 10 calls)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None,
            "launch_avg_ms": round(launch_avg, 5),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }


def bench_sparse(a, cfg):
    """Block-sparse forward on a seeded selection; MFMA roofline over the kept pairs."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    q, k, v = W.make_inputs(cfg, dev)
    rp, cols = W.sparse_selection(B, H, N, cfg["seed"], cfg["keep"])
    pairs = W.sparse_visible_pairs(N, rp, cols, B * H, cfg["causal"])
    row_ptr = torch.tensor(rp, dtype=torch.int32, device=dev)
    cols_t = torch.tensor(cols, dtype=torch.int32, device=dev)
    scale = 1.0 / d ** 0.5
    step = lambda: fa.forward_block_sparse(q, k, v, row_ptr, cols_t, causal=cfg["causal"], scale=scale)
    total_ms, per = time_launches(step, a.steps, a.warmup, stream, warm_ms=WARM_MS)
    ms = total_ms / a.steps
    flops = 4.0 * d * pairs
    launch_avg = sum(per) / len(per)
    dense = attention_flops(B, H, N, d, cfg["causal"])
    return {
        "metric": "block-sparse attention forward TFLOP/s over the kept (query, key) pairs",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"causal bf16 block-sparse attention forward, B={B} H={H} N={N} d={d}, "
                               f"blocks 256x64: first + diagonal + {cfg['keep']} of the rest",
                   "B": B, "H": H, "N": N, "d": d, "causal": bool(cfg["causal"]),
                   "nnz_blocks": int(cols.shape[0]), "kept_fraction_of_causal": round(flops / dense, 4)},
        "roofline": {
            "kernel": "fwd_bf16_kernel (block-sparse instance)",
            "bound": "mfma",
            "achieved": round(flops / (launch_avg * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (launch_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "launch_avg_ms": round(launch_avg, 4),
            "algorithmic_flops_per_launch": flops,
        },
    }


def bench_fp8(a, cfg):
    """fp8 (e4m3) forward at the causal headline shape; fp8 MFMA roofline."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    (q, k, v), (qd, kd, vd) = W.make_fp8_inputs(cfg, dev)
    scale = 1.0 / d ** 0.5
    step = lambda: fa.forward_fp8(q, k, v, qd, kd, vd, causal=cfg["causal"], scale=scale)
    total_ms, per = time_launches(step, a.steps, a.warmup, stream, warm_ms=WARM_MS)
    ms = total_ms / a.steps
    flops = attention_flops(B, H, N, d, cfg["causal"])
    launch_avg = sum(per) / len(per)
    achieved = flops / (launch_avg * 1e-3) / 1e12
    return {
        "metric": "attention TFLOP/s fwd at N=16K d=128, fp8 (e4m3) inputs; % of fp8 MFMA peak",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"causal fp8 (e4m3) attention forward, B={B} H={H} N={N} d={d}, bf16 O",
                   "B": B, "H": H, "N": N, "d": d, "causal": bool(cfg["causal"])},
        "roofline": {
            "kernel": "fwd_fp8_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": None,
            "launch_avg_ms": round(launch_avg, 4),
            "algorithmic_flops_per_launch": flops,
        },
    }


def _fwd_entry(ms_list, flops):
    avg = sum(ms_list) / len(ms_list)
    tf = flops / (avg * 1e-3) / 1e12
    return {"launch_avg_ms": round(avg, 4), "median_ms": round(_median(ms_list), 4),
            "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_other_configs(a, dev, stream, headline_launch_avg_ms):
    """Configurations 2, 4 and 5 and the rising-score worst case, timed like the headline."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    steps, warmup = max(5, min(a.steps, 20)), max(1, min(a.warmup, 5))
    out = {}
    # 2: non-causal B8 H32 N2048 with Q x4; its 0.5 GB of inputs and output fit the
    # memory-side cache, so it is timed warm (back to back) and cold (a 512 MiB
    # write between launches)
    cfg = W.config(2)
    q, k, v = W.make_inputs(cfg, dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fl = attention_flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"])
    fwd = lambda: fa.forward(q, k, v, causal=cfg["causal"], scale=cfg["scale"], out=o, lse=lse)
    _, warm = time_launches(fwd, steps, warmup, stream, warm_ms=WARM_MS)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    _, cold = time_launches(fwd, steps, warmup, stream, between=lambda: flush.fill_(1), warm_ms=WARM_MS)
    out["config2"] = {"workload": "non-causal bf16 forward, B=8 H=32 N=2048 d=128, Q x4",
                      "flops": fl, "warm": _fwd_entry(warm, fl), "cold": _fwd_entry(cold, fl)}
    del q, k, v, o, lse, flush
    # 4: causal B1 H8 N100000 (ragged tail)
    cfg = W.config(4)
    q, k, v = W.make_inputs(cfg, dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fl = attention_flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"])
    _, per = time_launches(lambda: fa.forward(q, k, v, causal=True, scale=cfg["scale"], out=o, lse=lse),
                           steps, warmup, stream, warm_ms=WARM_MS)
    out["config4"] = {"workload": "causal bf16 forward, B=1 H=8 N=100000 d=128", "flops": fl,
                      **_fwd_entry(per, fl)}
    del q, k, v, o, lse
    # 5: the backward of causal B4 H16 N4096 (5 products, 10 N^2 d per head, halved)
    cfg = W.config(5)
    q, k, v, do = W.make_inputs(cfg, dev, with_do=True)
    o, lse = fa.forward(q, k, v, causal=True, scale=cfg["scale"])
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    ws = torch.empty(fa.backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    fl = 2.5 * attention_flops(B, H, N, d, True)
    bwd = lambda: fa.backward(q, k, v, o, do, lse, causal=True, scale=cfg["scale"], workspace=ws)
    _, warm = time_launches(bwd, steps, warmup, stream, warm_ms=WARM_MS)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    _, cold = time_launches(bwd, steps, warmup, stream, between=lambda: flush.fill_(1), warm_ms=WARM_MS)
    out["config5_backward"] = {"workload": "backward of causal bf16 attention, B=4 H=16 N=4096 d=128 "
                                           "(dq, dk, dv; 3 kernels)",
                               "flops": fl, "warm": _fwd_entry(warm, fl), "cold": _fwd_entry(cold, fl)}
    del q, k, v, do, o, lse, ws, flush
    # worst case of the fast pass: rising scores at the headline shape
    cfg = W.RISING_WORKLOADS["rising"]
    q, k, v = W.make_rising_inputs(cfg, dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fl = attention_flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], True)
    _, per = time_launches(lambda: fa.forward(q, k, v, causal=True, out=o, lse=lse), steps, warmup, stream,
                           warm_ms=WARM_MS)
    e = _fwd_entry(per, fl)
    out["worst_case"] = {
        "workload": f"causal bf16 forward, B=8 H=32 N=16384 d=128, scores rising by {cfg['slope']:g} (log2) "
                    "per 64 keys: the fast pass's row-sum bound fails in every query block, about every third "
                    "tile, each time rescaled in place",
        **e, "over_normal_inputs": round(e["launch_avg_ms"] / headline_launch_avg_ms, 4)}
    del q, k, v, o, lse
    return out


def bench_widened(a):
    """The widened rows in the same invocation, briefly: decode at the 100K-token
    and 16K caches, the fp8 forward, the block-sparse forward and the forward
    with 8 shared key/value heads, each as its own `--workload` line would
    time it (fewer steps), reduced to its figures and roofline fraction."""
    import torch

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    sub = argparse.Namespace(**vars(a))
    sub.steps, sub.warmup = max(5, min(a.steps, 10)), 2
    out = {}

    def keep(name, r):
        out[name] = {"workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
                     "ms_per_step": r["ms_per_step"], "roofline_frac": r["roofline"]["frac"],
                     "roofline_peak": r["roofline"]["peak"], "launch_avg_ms": r["roofline"]["launch_avg_ms"]}

    for name, fn in (("decode_long", lambda: bench_decode(sub, W.DECODE_WORKLOADS["decode_long"])),
                     ("decode", lambda: bench_decode(sub, W.DECODE_WORKLOADS["decode"])),
                     ("fp8", lambda: bench_fp8(sub, W.FP8_WORKLOADS["fp8"])),
                     ("sparse", lambda: bench_sparse(sub, W.SPARSE_WORKLOADS["sparse"]))):
        try:
            keep(name, fn())
        except RuntimeError as e:
            out[name] = {"error": str(e)}
        torch.cuda.empty_cache()
    try:
        cfg = W.gqa_config("gqa")
        dev = torch.device("cuda:0")
        q, k, v = W.make_inputs(cfg, dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fl = attention_flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"])
        _, per = time_launches(lambda: fa.forward(q, k, v, causal=cfg["causal"], scale=cfg["scale"], out=o, lse=lse),
                               sub.steps, sub.warmup, torch.cuda.current_stream(dev), warm_ms=WARM_MS)
        e = _fwd_entry(per, fl)
        out["gqa"] = {"workload": f"causal bf16 forward, B={cfg['B']} H={cfg['H']} Hkv={cfg['Hkv']} "
                                  f"N={cfg['N']} d={cfg['d']}", "value": e["tflops"], "unit": "TFLOP/s",
                      "ms_per_step": e["launch_avg_ms"], "roofline_frac": e["frac_of_peak"],
                      "roofline_peak": PEAK_BF16_TFLOPS, "launch_avg_ms": e["launch_avg_ms"]}
        del q, k, v, o, lse
    except RuntimeError as e:
        out["gqa"] = {"error": str(e)}
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- main


def main():
    a = parse()
    if a.stats_summary:
        print(stats_summary(*a.stats_summary), end="")
        return
    if a.ceiling_summary:
        ceiling_summary(*a.ceiling_summary)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if a.profile_child:
        profile_child(a)
        return

    headline = not a.workload and a.config == 3
    # (pages the image in; imports touch no GPU)
    import torch  # noqa: F401

    prof_dirs = None
    if headline and not a.no_profile:
        # the child passes run first, one after another: this process has not
        # touched the GPU (and never re-executes itself)
        outdir = os.path.abspath(a.profile_out) if a.profile_out else tempfile.mkdtemp(prefix="fa_bench_", dir="/tmp")
        paths, errors = {}, []
        rocprof = rocprof_bin()
        if rocprof is None:
            errors.append("rocprofv3 not found")
        else:
            for kind in ("trace", "sq", "tcc"):
                os.makedirs(os.path.join(outdir, kind), exist_ok=True)
                paths[kind], err = run_one_child(kind, outdir, rocprof)
                errors += err
        prof_dirs = {"dir": outdir, "paths": paths, "errors": errors}

    import exact_tiled_attention_38_amd as fa
    from exact_tiled_attention_38_amd import workloads as W

    if a.workload and a.workload.startswith("decode"):
        print(json.dumps(bench_decode(a, W.DECODE_WORKLOADS[a.workload])), flush=True)
        return
    if a.workload == "fp8":
        print(json.dumps(bench_fp8(a, W.FP8_WORKLOADS["fp8"])), flush=True)
        return
    if a.workload == "sparse":
        print(json.dumps(bench_sparse(a, W.SPARSE_WORKLOADS["sparse"])), flush=True)
        return
    if a.workload == "gemm_ceiling":
        print(json.dumps(bench_gemm_ceiling(a)), flush=True)
        return
    if a.workload == "rising":
        cfg = dict(W.RISING_WORKLOADS["rising"], scale=1.0 / 128 ** 0.5, passes=("fwd",))
    else:
        cfg = W.gqa_config(a.workload) if a.workload else W.config(a.config)
    B, H, N, d, causal, scale = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"], cfg["scale"]
    Hkv = cfg.get("Hkv", H)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if a.workload == "rising":
        q, k, v = W.make_rising_inputs(cfg, dev)
        do = None
    else:
        q, k, v, do = W.make_inputs(cfg, dev, with_do=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    log("timing the forward")
    fwd = lambda: fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    props = torch.cuda.get_device_properties(dev)
    sampler = ClockSampler(props)
    total_ms, per = time_launches(fwd, a.steps, a.warmup, stream, sampler=sampler)
    ms = total_ms / a.steps
    flops = attention_flops(B, H, N, d, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    per_sorted = sorted(per)
    launch_avg = sum(per) / len(per)

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("causal " if causal else "") + f"bf16 attention forward, B={B} H={H} "
                        + (f"Hkv={Hkv} " if Hkv != H else "") + f"N={N} d={d}"
                        + (", rising scores" if a.workload == "rising" else ""),
            "B": B, "H": H, "N": N, "d": d, "causal": bool(causal), "scale": scale,
            "cu_count": props.multi_processor_count,
            "device": torch.cuda.get_device_name(dev),
            "gcn_arch": getattr(props, "gcnArchName", None),
        },
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "median_ms": round(per_sorted[len(per) // 2], 4),
        "min_ms": round(per_sorted[0], 4),
        "roofline": {
            "kernel": "fwd_bf16_kernel",
            "bound": "mfma",
            "achieved": round(flops / (launch_avg * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (launch_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "launch_avg_ms": round(launch_avg, 4),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": algorithmic_fwd_bytes(B, H, N, d, Hkv),
        },
    }
    if Hkv != H:
        result["config"]["Hkv"] = Hkv
    result["clocks"] = sampler.summary()

    if prof_dirs is not None:
        prof = headline_profile(prof_dirs["paths"], prof_dirs["errors"], launch_avg)
        t = prof.get("traffic")
        # a figure below the bytes the kernel must move cannot be what it moved
        if t and t["fwd_traffic_bytes"] >= result["roofline"]["algorithmic_bytes_per_launch"]:
            result["roofline"]["traffic"] = round(t["fwd_traffic_bytes"])
            result["roofline"]["achieved_hbm_gbs"] = round(t["fwd_traffic_bytes"] / (launch_avg * 1e-3) / 1e9, 1)
            result["roofline"]["traffic_source"] = ("32 x (TCC_EA0_RDREQ_DRAM_32B + TCC_EA0_WRREQ_WRITE_DRAM_32B) "
                                                    "per launch, copy-calibrated, in this invocation")
        result["profile"] = prof
        if a.profile_out:
            write_profile_records(prof_dirs["dir"], prof_dirs["paths"], prof, launch_avg)
        else:
            shutil.rmtree(prof_dirs["dir"], ignore_errors=True)

    if headline:
        log("timing the vendor GEMM")
        g_ms, g_tf = time_vendor_gemm(min(a.steps, 10), 2)
        result["ceiling"] = {
            "vendor_bf16_gemm_tflops": round(g_tf, 2),
            "workload": f"torch.matmul bf16 {GEMM_N}x{GEMM_N}x{GEMM_N}",
            "frac_of_vendor_gemm": round(result["roofline"]["achieved"] / g_tf, 4),
        }
        ceil = read_ceiling()
        if ceil:
            result["ceiling"].update({"record_engine_clock_ghz": float(ceil["engine_clock_ghz"]),
                                      "record_mfma_busy_frac": float(ceil["mfma_busy_frac"]),
                                      "source": os.path.relpath(CEILING_FILE, ROOT)})

    if not a.no_bwd and do is not None and "fwd+bwd" in cfg["passes"]:
        log("timing fwd+bwd")
        ws = torch.empty(fa.backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        try:
            def fwd_bwd():
                fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
                fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, workspace=ws)

            fb_total, _ = time_launches(fwd_bwd, a.steps, a.warmup, stream)
            fb_ms = fb_total / a.steps
            fb_tf = 3.5 * flops / (fb_ms * 1e-3) / 1e12
            result["fwd_bwd"] = {"ms_per_step": round(fb_ms, 4), "tflops": round(fb_tf, 2),
                                 "frac_of_peak": round(fb_tf / PEAK_BF16_TFLOPS, 4),
                                 "flops": 3.5 * flops}
        except RuntimeError as e:
            result["fwd_bwd"] = {"error": str(e)}
        del ws

    if headline and not a.no_extra:
        log("timing the other configurations and the worst case")
        result["configs"] = bench_other_configs(a, dev, stream, launch_avg)
        result["worst_case"] = result["configs"].pop("worst_case")
        log("timing the widened rows (decode, fp8, block-sparse, shared heads)")
        result["widened"] = bench_widened(a)

    if not a.no_cpu_baseline and a.workload != "rising":
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, q, k, v, a.cpu_seconds)

    print(json.dumps(result), flush=True)


def run_one_child(kind, outdir, rocprof):
    """One rocprofv3 child pass; returns (csv path or None, errors)."""
    cmd = child_command(kind, outdir, rocprof)
    env = dict(os.environ, TMPDIR="/tmp", BENCH_CHILD_DIR=os.path.join(outdir, kind))
    log(f"profile pass {kind}")
    t0 = time.time()
    with open(os.path.join(outdir, f"{kind}.log"), "w") as fh:
        p = subprocess.Popen(cmd, cwd="/tmp", env=env, stdout=fh, stderr=subprocess.STDOUT,
                             start_new_session=True)
        try:
            rc = p.wait(timeout=CHILD_TIMEOUT_S)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, 9)
            p.wait()
            rc = "timeout"
    name = "run_kernel_trace.csv" if kind == "trace" else "run_counter_collection.csv"
    path = os.path.join(outdir, kind, name)
    done = os.path.exists(os.path.join(outdir, kind, "child_done"))
    log(f"profile pass {kind}: {time.time() - t0:.1f} s, exit status {rc}")
    # rocprofv3 may end with a fault of its own after the program finished and
    # its files are whole: the program's completion marker decides
    if done and os.path.exists(path):
        return path, ([] if rc == 0 else [f"{kind}: rocprofv3 exit status {rc} after the program completed"])
    return None, [f"{kind}: no complete output (exit status {rc})"]


if __name__ == "__main__":
    main()
