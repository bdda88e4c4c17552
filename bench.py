"""Benchmark of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--config 3]

Workload: the causal bf16 forward at B=8, H=32, N=16384, d=128 (the "16K
tokens x 32 heads x batch 8" shape of "FlashAttention" (tensorlab.fun), Beat
01), inputs i.i.d. N(0, 1) from a fixed seed, resident in HBM before timing.
A step is one fa_forward call over the whole batch; `value` is attention
TFLOP/s = 4 N^2 d B H (halved for causal) / step time. The fwd+bwd pass at
the same shape (fa_forward + fa_backward, 3.5x the forward FLOPs) is timed
as well and reported under "fwd_bwd".

Prints exactly one JSON line on stdout. The roofline block prices the
forward kernel against the MI355X dense-bf16 matrix peak (2516.6 TFLOP/s:
256 CUs x 4096 FLOP/clk x 2.4 GHz); per-launch durations come from HIP
events recorded on the stream the kernel runs on. cpu_baseline times the fp64
CPU oracle on a bounded sample of rows of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd (and fwd+bwd) at N=16K d=128 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU * 4096 FLOP/clk/CU * 2.4 GHz, dense bf16
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 matrix peak, twice the bf16 one


def attention_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload configuration id (3 = headline)")
    ap.add_argument("--workload", choices=["gqa", "mqa", "decode", "decode_gqa", "decode_long", "sparse", "fp8",
                                           "gemm_ceiling"],
                    help="instead of --config: the same causal 16K shape with 8 (gqa) or 1 (mqa) "
                         "key/value heads shared by the 32 query heads, or a decode workload (one "
                         "query per head against a 16K or 100K-token cache), or the block-sparse "
                         "forward on the causal 16K shape (first block + diagonal + 1/8 of the rest), "
                         "or the fp8 (e4m3) forward on the causal 16K shape, or (context, not the "
                         "library) the vendor bf16 GEMM torch.matmul at 16384^3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the fwd+bwd timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (reference for the HBM byte counters)")
    ap.add_argument("--counters-summary", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                    help="no GPU work: turn one rocprofv3 --pmc --kernel-trace run of `bench.py --no-bwd` "
                         "into the forward's counter record under profiles/ (MFMA busy, LDS bank "
                         "conflicts, engine clock)")
    ap.add_argument("--ceiling-summary", nargs=2, metavar=("COUNTER_CSV", "TRACE_CSV"),
                    help="no GPU work: turn one rocprofv3 --pmc --kernel-trace run of "
                         "`bench.py --workload gemm_ceiling` into the GEMM ceiling record under profiles/")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --calibration-copy --no-bwd` into the traffic record under profiles/")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_traffic_causal_b8h32n16384d128.md")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_counters_causal_b8h32n16384d128.md")
CEILING_FILE = os.path.join(ROOT, "profiles", "gemm_bf16_ceiling_m16384n16384k16384.md")
GEMM_N = 16384
CEILING_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
N_XCD, N_CU, SIMD_PER_CU, FLOP_PER_CLK_CU = 8, 256, 4, 4096
COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
            "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"]
FWD_SOURCES = ["fa_fwd_bf16.hip", "fa_device.h"]
COPY_BYTES = 1 << 30


def fwd_source_hash():
    """sha256 over the forward kernel's sources: a traffic figure is only
    reported for the kernel it was measured on."""
    import hashlib

    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_38_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_record(path):
    """key: value lines of a committed record, or {} when there is none or the
    forward's sources changed since it was taken."""
    try:
        rec = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
        return rec if rec.get("kernel_source_sha256") == fwd_source_hash() else {}
    except OSError:
        return {}


def counters_summary(counter_csv, trace_csv, out=None):
    """Write the forward's counter record from one --pmc --kernel-trace run.

    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the engine clock during the
    kernel is GRBM_GUI_ACTIVE / 8 / duration; MFMA busy is
    SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); the LDS bank-conflict
    rate is SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    import csv

    vals = {}
    for r in csv.DictReader(open(counter_csv)):
        if "fwd_bf16_kernel" in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    durs = []
    for r in csv.DictReader(open(trace_csv)):
        if "fwd_bf16_kernel" in r["Kernel_Name"]:
            durs.append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
    mean = lambda k: sum(vals[k]) / len(vals[k])
    dur = sum(durs) / len(durs)
    cycles = mean("GRBM_GUI_ACTIVE") / N_XCD
    sclk = cycles / dur / 1e9
    mfma = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * N_CU * SIMD_PER_CU)
    conf = mean("SQ_LDS_BANK_CONFLICT") / max(mean("SQ_LDS_IDX_ACTIVE"), 1.0)
    adj_peak = N_CU * FLOP_PER_CLK_CU * sclk * 1e9 / 1e12
    lines = [
        "# Counters of fwd_bf16_kernel, causal bf16 attention forward B=8 H=32 N=16384 d=128, one MI355X",
        "# Command (from the repository root, cd /tmp && export TMPDIR=/tmp first):",
        "#   rocprofv3 --pmc " + " ".join(COUNTERS) + " --kernel-trace --output-format csv -d <out>/ctr -o run \\",
        "#       -- python3 <repo>/bench.py --steps 2 --warmup 0 --no-bwd --no-cpu-baseline",
        "#   python bench.py --counters-summary <out>/ctr/run_counter_collection.csv <out>/ctr/run_kernel_trace.csv",
        "# GRBM_GUI_ACTIVE is summed over the 8 XCDs: engine clock = GRBM_GUI_ACTIVE / 8 / kernel duration.",
        "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 256 CU x 4 SIMD).",
        "# (the profiled launches run somewhat slower than unprofiled ones; the fractions are what they measure)",
        f"kernel_source_sha256: {fwd_source_hash()}",
        f"launches: {len(durs)}",
        f"duration_ms: {dur * 1e3:.3f}",
        f"engine_clock_ghz: {sclk:.3f}",
        f"clock_adjusted_peak_tflops: {adj_peak:.1f}",
        f"mfma_busy_frac: {mfma:.4f}",
        f"lds_bank_conflict_frac: {conf:.4f}",
        f"mfma_instructions: {mean('SQ_INSTS_MFMA'):.4g}",
        "# each v_mfma_f32_32x32x16_bf16 is 32 x 32 x 16 x 2 = 32768 FLOPs; against the algorithmic count the",
        "# ratio is 1 + the work of masked diagonal/tail tiles and of the even-count padding step",
        f"mfma_flops_over_algorithmic: {mean('SQ_INSTS_MFMA') * 32768 / attention_flops(8, 32, 16384, 128, True):.4f}",
        f"valu_instructions: {mean('SQ_INSTS_VALU'):.4g}",
        f"lds_instructions: {mean('SQ_INSTS_LDS'):.4g}",
    ]
    with open(out or COUNTERS_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def time_vendor_gemm(steps, warmup):
    """The vendor's bf16 GEMM (torch.matmul -> hipBLASLt) at 16384^3 on the same
    part: what a dense matrix product reaches here under the same power and
    clock limits. Context for the attention kernels' roofline, not a library
    path. Returns (ms per product, TFLOP/s)."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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

    ms, tflops = time_vendor_gemm(a.steps, a.warmup)
    dev = torch.device("cuda:0")
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


def read_traffic(path=None):
    """HBM bytes per forward launch from the committed counter record, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        rec = {}
        for line in open(path or TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
        if rec.get("kernel_source_sha256") != fwd_source_hash():
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def pmc_summary(fetch_csv, write_csv, out=None):
    """Write the traffic record from a FETCH_SIZE run and a WRITE_SIZE run.

    Both counters are in KiB per dispatch. Each is scaled by what it reads for
    a plain device copy of COPY_BYTES (which reads and writes COPY_BYTES), so
    the result is in bytes as that copy defines them."""
    import csv

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    pick = lambda d, pat: [v for k, vs in d.items() if pat(k) for v in vs]
    is_copy = lambda k: "copy" in k.lower() and "fwd_bf16" not in k
    is_fwd = lambda k: "fwd_bf16_kernel" in k
    cf, cw = max(pick(f, is_copy)), max(pick(w, is_copy))  # the 1 GiB copy is the largest copy
    ff, fw = pick(f, is_fwd), pick(w, is_fwd)
    fetch_scale = COPY_BYTES / (cf * 1024.0)
    write_scale = COPY_BYTES / (cw * 1024.0)
    fk, wk = sum(ff) / len(ff), sum(fw) / len(fw)
    traffic = fk * 1024.0 * fetch_scale + wk * 1024.0 * write_scale
    lines = [
        "# HBM traffic of fwd_bf16_kernel, causal bf16 attention forward B=8 H=32 N=16384 d=128",
        "# Two counter runs on one MI355X, from the repository root (cd /tmp && export TMPDIR=/tmp first):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- python3 <repo>/bench.py --steps 1 --warmup 0 --no-bwd --no-cpu-baseline --calibration-copy",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- python3 <repo>/bench.py --steps 1 --warmup 0 --no-bwd --no-cpu-baseline --calibration-copy",
        "#   python bench.py --pmc-summary <out>/fetch/run_counter_collection.csv <out>/write/run_counter_collection.csv",
        "# Counters are KiB per dispatch; each is scaled by the reading of a plain 1 GiB device copy",
        "# (1 GiB read + 1 GiB written) in the same run.",
        "# Caveat: K and V reach the forward by direct-to-LDS loads, and for the decode kernel, which reads",
        "# every K/V byte exactly once by the same loads, FETCH_SIZE reads half of those bytes; the fetch",
        "# figure below is therefore a lower bound on the bytes the forward pulls through the L2.",
        f"kernel_source_sha256: {fwd_source_hash()}",
        f"copy_bytes: {COPY_BYTES}",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_scale: {fetch_scale:.4f}",
        f"write_scale: {write_scale:.4f}",
        f"fwd_fetch_kib_per_launch: {fk:.1f}",
        f"fwd_write_kib_per_launch: {wk:.1f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"algorithmic_bytes_per_launch: {algorithmic_fwd_bytes(8, 32, 16384, 128):.0f}",
    ]
    with open(out or TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def algorithmic_fwd_bytes(B, H, N, d, Hkv=None):
    """Q, K, V read once and O written once (bf16), lse written once (fp32)."""
    Hkv = H if Hkv is None else Hkv
    return (2.0 * H + 2.0 * Hkv) * B * N * d * 2 + 4.0 * B * H * N


def time_launches(fn, steps, warmup, stream):
    """Run fn `warmup` times, then `steps` timed times. Returns (total ms, per-launch ms list)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end), [a.elapsed_time(b) for a, b in ev]


def cpu_baseline(cfg, q, k, v, target_s):
    """Time the fp64 oracle on whole rows of the same workload until ~target_s of work."""
    import numpy as np
    import torch

    import oracle
    from exact_tiled_attention_38_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
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
        "cores": int(cores),
        "cpu_model": cpu_model,
        "extrapolated_full_workload_seconds": round(attention_flops(B, H, N, d, causal) / rate, 1),
        "kind": "oracle",
        "sample": f"fp64 one-shot oracle on {len(rows)} seeded rows (full score rows) of each of {done} heads "
                  f"of the same workload; rate = algorithmic attention FLOPs of those rows "
                  f"(4 d x visible keys) / {elapsed:.1f} s",
        "seconds": elapsed,
    }


def decode_bytes(cfg):
    """Algorithmic bytes of one decode call: K and V read once, Q read, O and lse written."""
    B, H, Hkv, Nq, Nk, d = (cfg[x] for x in ("B", "H", "Hkv", "Nq", "Nk", "d"))
    return 2.0 * B * Hkv * Nk * d * 2 + 2.0 * B * H * Nq * d * 2 + 4.0 * B * H * Nq


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
    total_ms, per = time_launches(step, a.steps, a.warmup, stream)
    ms = total_ms / a.steps
    nbytes = decode_bytes(cfg)
    launch_avg = sum(per) / len(per)
    gbs = nbytes / (ms * 1e-3) / 1e9
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
        "roofline": {
            "kernel": "decode_kernel + merge_kernel (one fa_decode call)",
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
    total_ms, per = time_launches(step, a.steps, a.warmup, stream)
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
    total_ms, per = time_launches(step, a.steps, a.warmup, stream)
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


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.counters_summary:
        counters_summary(*a.counters_summary)
        return
    if a.ceiling_summary:
        ceiling_summary(*a.ceiling_summary)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

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
    cfg = W.gqa_config(a.workload) if a.workload else W.config(a.config)
    B, H, N, d, causal, scale = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"], cfg["scale"]
    Hkv = cfg.get("Hkv", H)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    q, k, v, do = W.make_inputs(cfg, dev, with_do=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if a.calibration_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    fwd = lambda: fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    total_ms, per = time_launches(fwd, a.steps, a.warmup, stream)
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
                        + (f"Hkv={Hkv} " if Hkv != H else "") + f"N={N} d={d}",
            "B": B, "H": H, "N": N, "d": d, "causal": bool(causal), "scale": scale,
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

    result["config"]["cu_count"] = torch.cuda.get_device_properties(dev).multi_processor_count
    result["config"]["device"] = torch.cuda.get_device_name(dev)
    if a.config == 3 and not a.workload:
        result["roofline"]["traffic"] = read_traffic()
        if result["roofline"]["traffic"]:
            result["roofline"]["achieved_hbm_gbs"] = round(
                result["roofline"]["traffic"] / (launch_avg * 1e-3) / 1e9, 1)
        rec = read_record(COUNTERS_FILE)
        if rec:
            # counters of the same kernel (profiled launches), from the committed record
            result["counters"] = {
                "mfma_busy_frac": float(rec["mfma_busy_frac"]),
                "lds_bank_conflict_frac": float(rec["lds_bank_conflict_frac"]),
                "engine_clock_ghz": float(rec["engine_clock_ghz"]),
                "clock_adjusted_peak_tflops": float(rec["clock_adjusted_peak_tflops"]),
                "frac_of_clock_adjusted_peak": round(
                    result["roofline"]["achieved"] / float(rec["clock_adjusted_peak_tflops"]), 4),
                "mfma_flops_over_algorithmic": float(rec["mfma_flops_over_algorithmic"]),
                "source": os.path.relpath(COUNTERS_FILE, ROOT),
            }
        # the vendor's dense bf16 GEMM on this part, timed here the same way: what
        # a matrix product without softmax work reaches under the same limits
        # (its clock and MFMA busy fraction come from the committed record)
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

    if not a.no_bwd and "fwd+bwd" in cfg["passes"]:
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

    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, q, k, v, a.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
