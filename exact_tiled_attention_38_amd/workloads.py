"""Seeded synthetic workloads: the five configurations, input generators,
row samplers and the bookkeeping probe inputs.

This module draws and lays out inputs only; it computes nothing of the
attention method. Tests and the benchmark feed the same tensors to the HIP
library and (read back to the host) to the CPU oracle.

Values: i.i.d. N(0, 1), drawn as fp32 with a seeded torch.Generator on the
device the tensors live on, then rounded to bf16 (fp32 kept for the fp32
configuration). The oracle always reads back the exact values the GPU used,
so parity does not depend on the generator being portable across devices.
Seeds are 3800 + configuration id for tensors and +1 for row sampling.
"""

import numpy as np
import torch

# Shapes from the pages: 16K tokens x 32 heads x batch 8 is the "256 GiB of
# scores and probabilities per layer" example of "FlashAttention"
# (tensorlab.fun), Beat 01; a 100,000-token head with d = 128 is the 20 GB
# score-matrix example of "FlashAttention — how 100K-token attention fits in
# memory" (llmdaily.org, day 19).
CONFIGS = {
    1: dict(name="tiny_exact_f32_b1h1n256d64", B=1, H=1, N=256, d=64, dtype="f32", causal=False,
            q_mult=1.0, seed=3801, passes=("fwd",)),
    2: dict(name="fwd_noncausal_bf16_b8h32n2048d128_q4", B=8, H=32, N=2048, d=128, dtype="bf16",
            causal=False, q_mult=4.0, seed=3802, passes=("fwd",)),
    3: dict(name="fwd_causal_bf16_b8h32n16384d128", B=8, H=32, N=16384, d=128, dtype="bf16",
            causal=True, q_mult=1.0, seed=3803, passes=("fwd", "fwd+bwd")),
    4: dict(name="fwd_causal_bf16_b1h8n100000d128", B=1, H=8, N=100000, d=128, dtype="bf16",
            causal=True, q_mult=1.0, seed=3804, passes=("fwd",)),
    5: dict(name="bwd_causal_bf16_b4h16n4096d128", B=4, H=16, N=4096, d=128, dtype="bf16",
            causal=True, q_mult=1.0, seed=3805, passes=("fwd", "bwd")),
}


# Shared key/value heads: the causal 16K-token shape above with 32 query heads
# over 8 key/value heads (groups of 4), and a multi-query variant (one
# key/value head). The pages give no shared-head workload; these keep the
# headline shape and vary only the head sharing.
GQA_WORKLOADS = {
    "gqa": dict(name="fwd_causal_bf16_b8h32kv8n16384d128", B=8, H=32, Hkv=8, N=16384, d=128,
                dtype="bf16", causal=True, q_mult=1.0, seed=3811),
    "mqa": dict(name="fwd_causal_bf16_b8h32kv1n16384d128", B=8, H=32, Hkv=1, N=16384, d=128,
                dtype="bf16", causal=True, q_mult=1.0, seed=3812),
}


# Decode: one new query per head against a cached sequence. The first two
# keep the headline shape (batch 8, 32 query heads, 16K cached tokens,
# d = 128) with 32 or 8 key/value heads; the third is the 100,000-token
# single-sequence length of the long-context page with 8 heads. Queries sit
# at the end of the sequence (causal; with one query that masks nothing).
DECODE_WORKLOADS = {
    "decode": dict(name="decode_bf16_b8h32kv32nq1nk16384d128", B=8, H=32, Hkv=32, Nq=1, Nk=16384, d=128,
                   causal=True, seed=3821),
    "decode_gqa": dict(name="decode_bf16_b8h32kv8nq1nk16384d128", B=8, H=32, Hkv=8, Nq=1, Nk=16384, d=128,
                       causal=True, seed=3822),
    "decode_long": dict(name="decode_bf16_b1h8kv8nq1nk100000d128", B=1, H=8, Hkv=8, Nq=1, Nk=100000, d=128,
                        causal=True, seed=3823),
}


# Block-sparse selection on the causal headline shape (B8 H32 N16384 d128):
# each 256-row query block keeps the first key block (64 keys), the four key
# blocks under its own rows, and every other key block before it with
# probability 1/8, drawn per (b, h, query block) from a fixed seed.
SPARSE_WORKLOADS = {
    "sparse": dict(name="fwd_block_sparse_causal_bf16_b8h32n16384d128_p8", B=8, H=32, Hkv=32, N=16384,
                   d=128, dtype="bf16", causal=True, q_mult=1.0, seed=3831, keep=0.125),
}


def sparse_selection(B, H, N, seed, keep, block_m=256, block_n=64):
    """CSR selection (row_ptr, cols) as int32 numpy arrays, rows ordered (b, h, query block).

    Query block r keeps key block 0, the key blocks covering its own rows,
    and each earlier key block with probability `keep` (seeded)."""
    rng = np.random.default_rng(seed)
    n_qb, n_kb = -(-N // block_m), -(-N // block_n)
    per = block_m // block_n
    row_ptr, cols = [0], []
    for _ in range(B * H):
        for r in range(n_qb):
            diag = set(range(r * per, min(n_kb, (r + 1) * per)))
            earlier = np.arange(0, r * per)
            chosen = set(earlier[rng.random(earlier.shape[0]) < keep].tolist()) | diag | {0}
            cols.extend(sorted(chosen))
            row_ptr.append(len(cols))
    return np.array(row_ptr, dtype=np.int32), np.array(cols, dtype=np.int32)


def sparse_visible_pairs(N, row_ptr, cols, n_heads, causal, block_m=256, block_n=64):
    """Number of (query, key) pairs the selection keeps, over all heads (for FLOP counts)."""
    n_qb = -(-N // block_m)
    total = 0
    r_idx = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    qb = r_idx % n_qb
    q_lo, q_hi = qb * block_m, np.minimum(N, (qb + 1) * block_m)
    k_lo, k_hi = cols.astype(np.int64) * block_n, np.minimum(N, (cols.astype(np.int64) + 1) * block_n)
    if not causal:
        total = int(np.sum((q_hi - q_lo) * (k_hi - k_lo)))
    else:
        # pairs with k <= q inside each block rectangle: per query row i,
        # clip(min(i + 1, j1) - j0, 0), summed over the rows (in chunks of blocks)
        off = np.arange(block_m)
        for c0 in range(0, q_lo.shape[0], 8192):
            i = q_lo[c0:c0 + 8192, None] + off[None, :]
            valid = i < q_hi[c0:c0 + 8192, None]
            cnt = np.clip(np.minimum(i + 1, k_hi[c0:c0 + 8192, None]) - k_lo[c0:c0 + 8192, None], 0, None)
            total += int((cnt * valid).sum())
    return total


# fp8 (e4m3) forward on the causal headline shape: N(0, 1) values quantised
# per tensor with the factor amax / 448 (the largest e4m3 value).
FP8_WORKLOADS = {
    "fp8": dict(name="fwd_fp8_causal_b8h32n16384d128", B=8, H=32, Hkv=32, N=16384, d=128, causal=True,
                seed=3841),
}
E4M3_MAX = 448.0


def quantize_e4m3(x):
    """Per-tensor e4m3 codes of x and the dequantisation factor (x ~ codes * factor)."""
    factor = float(x.abs().max()) / E4M3_MAX
    factor = factor if factor > 0 else 1.0
    return (x / factor).to(torch.float8_e4m3fn), factor


def make_fp8_inputs(cfg, device, shape=None, kv_heads=None, seed=None):
    """Seeded e4m3 (q, k, v) and their factors (qd, kd, vd): N(0, 1) drawn in fp32, quantised per tensor."""
    B, H, N, d = shape or (cfg["B"], cfg["H"], cfg["N"], cfg["d"])
    Hkv = kv_heads or cfg.get("Hkv") or H
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg["seed"] if seed is None else seed)
    out, factors = [], []
    for heads in (H, Hkv, Hkv):
        x = _randn((B, heads, N, d), gen, device)
        codes, f = quantize_e4m3(x)
        out.append(codes.contiguous())
        factors.append(f)
        del x
    return tuple(out), tuple(factors)


def make_decode_inputs(cfg, device):
    """Seeded bf16 q [B, H, Nq, d] and k, v [B, Hkv, Nk, d], i.i.d. N(0, 1)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg["seed"])
    out = []
    for shape in ((cfg["B"], cfg["H"], cfg["Nq"], cfg["d"]), (cfg["B"], cfg["Hkv"], cfg["Nk"], cfg["d"]),
                  (cfg["B"], cfg["Hkv"], cfg["Nk"], cfg["d"])):
        x = _randn(shape, gen, device)
        out.append(x.to(torch.bfloat16).contiguous())
        del x
    return tuple(out)


def gqa_config(kind):
    c = dict(GQA_WORKLOADS[kind])
    c["id"] = kind
    c["scale"] = 1.0 / float(np.sqrt(c["d"]))
    c["passes"] = ("fwd", "fwd+bwd")
    return c


def config(cid):
    c = dict(CONFIGS[cid])
    c["id"] = cid
    c["scale"] = 1.0 / float(np.sqrt(c["d"]))
    return c


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_inputs(cfg, device, with_do=False, shape=None, seed=None, kv_heads=None):
    """Seeded (q, k, v[, do]) for a configuration dict (or an explicit shape).

    bf16 tensors are drawn in fp32 and rounded; config['q_mult'] multiplies q
    after drawing (x4 is exact in bf16). k and v get `kv_heads` heads
    (default: config['Hkv'], else as many as q). Returns contiguous tensors on
    device.
    """
    B, H, N, d = shape or (cfg["B"], cfg["H"], cfg["N"], cfg["d"])
    Hkv = kv_heads or cfg.get("Hkv") or H
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg["seed"] if seed is None else seed)
    out_dtype = torch.float32 if cfg.get("dtype") == "f32" else torch.bfloat16
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    tensors = []
    for name in names:
        x = _randn((B, Hkv if name in ("k", "v") else H, N, d), gen, device)
        if name == "q" and cfg.get("q_mult", 1.0) != 1.0:
            x.mul_(cfg["q_mult"])
        tensors.append(x.to(out_dtype).contiguous())
        del x
    return tuple(tensors)


def sample_rows(N, count, seed, tile=256):
    """Sorted distinct query rows: `count` uniform draws plus row 0, row N-1 and
    the first row of the last (possibly partial) tile of `tile` rows."""
    rng = np.random.default_rng(seed)
    base = rng.choice(N, size=min(count, N), replace=False)
    extra = np.array([0, N - 1, ((N - 1) // tile) * tile])
    return np.unique(np.concatenate([base, extra])).astype(np.int64)


def sample_heads(B, H, count, seed):
    """Seeded distinct (b, h) pairs."""
    rng = np.random.default_rng(seed)
    flat = rng.choice(B * H, size=min(count, B * H), replace=False)
    return [(int(f // H), int(f % H)) for f in sorted(flat)]


# ---------------------------------------------------------------- bookkeeping probes
#
# Inputs whose exact outputs follow from which keys each query row sees, so a
# test can check every row of a full-size configuration bit for bit:
#   count: Q = 0 and V = 1 make every visible score 0, so O = 1 and
#          exp(lse_i) = the number of visible keys.
#   max:   scale 1, Q_i = 32 * (4096, 64, 1, 0, ...) and
#          K_j = (floor(j / 4096) mod 64, floor(j / 64) mod 64, j mod 64, 0, ...)
#          give s_ij = 32 j exactly in fp32 (every factor is exact in bf16 and
#          every partial sum stays below 2^24); V_j[b] = bit b of j. The
#          largest visible key dominates by e^32 per step, so the bits of O_i
#          spell out the largest visible key index.
#   min:   the same with Q negated: O_i spells out the smallest visible key.

PROBE_BITS = 17  # 2^17 = 131072 > 100000


def probe_inputs(kind, B, H, N, d, device, dtype=torch.bfloat16):
    j = torch.arange(N, device=device, dtype=torch.int64)
    q = torch.zeros((N, d), device=device, dtype=torch.float32)
    k = torch.zeros((N, d), device=device, dtype=torch.float32)
    v = torch.zeros((N, d), device=device, dtype=torch.float32)
    if kind == "count":
        k.normal_(generator=torch.Generator(device=device).manual_seed(7))
        v.fill_(1.0)
    elif kind in ("max", "min"):
        sign = 1.0 if kind == "max" else -1.0
        q[:, 0], q[:, 1], q[:, 2] = sign * 32 * 4096, sign * 32 * 64, sign * 32
        k[:, 0] = ((j // 4096) % 64).float()
        k[:, 1] = ((j // 64) % 64).float()
        k[:, 2] = (j % 64).float()
        for bit in range(PROBE_BITS):
            v[:, bit] = ((j >> bit) & 1).float()
    else:
        raise ValueError(kind)
    expand = lambda x: x.to(dtype).expand(B, H, N, d).contiguous()
    return expand(q), expand(k), expand(v)


def probe_scale(kind, d):
    return 1.0 / float(np.sqrt(d)) if kind == "count" else 1.0


def decode_probe_index(o):
    """Key index spelled by the first PROBE_BITS columns of a probe output (0/1 each)."""
    bits = torch.round(o[..., :PROBE_BITS].float()).to(torch.int64)
    weights = (1 << torch.arange(PROBE_BITS, device=o.device, dtype=torch.int64))
    return (bits * weights).sum(-1)


# Probes with shared key/value heads and with queries at the end of a longer
# key sequence (decode). Key/value head g numbers its keys through the
# permutation r_g(j) = (j + off_g) mod Nk, off_g = 37 g mod Nk: the max and
# min probes' K_j spells r_g(j) (so s_ij = +-32 r_g(j) exactly), V_j spells
# the key index j in its first PROBE_BITS columns, and column PROBE_BITS of V
# holds g + 1. The row's output then spells the key index that maximises (or
# minimises) r_g over the row's visible keys, and its column PROBE_BITS reads
# g + 1: both the K and the V head of every query head are pinned exactly.
# The count probe is as above (Q = 0, V = 1), with column PROBE_BITS of V
# also g + 1, which every visible key then contributes with weight exactly 1.

def probe_key_order(g, Nk):
    """r_g(j) for j in range(Nk), as an int64 numpy array (a permutation of range(Nk))."""
    off = (37 * g) % Nk
    return (np.arange(Nk, dtype=np.int64) + off) % Nk


def probe_heads_inputs(kind, B, H, Hkv, Nq, Nk, d, device, dtype=torch.bfloat16, rotate=True):
    """(q [B, H, Nq, d], k [B, Hkv, Nk, d], v [B, Hkv, Nk, d]) for the shared-head probes above
    (rotate=False: r_g(j) = j for every head)."""
    if d <= PROBE_BITS:
        raise ValueError("probe needs d > PROBE_BITS")
    j = torch.arange(Nk, device=device, dtype=torch.int64)
    q = torch.zeros((Nq, d), device=device, dtype=torch.float32)
    if kind in ("max", "min"):
        sign = 1.0 if kind == "max" else -1.0
        q[:, 0], q[:, 1], q[:, 2] = sign * 32 * 4096, sign * 32 * 64, sign * 32
    elif kind != "count":
        raise ValueError(kind)
    ks, vs = [], []
    for g in range(Hkv):
        k = torch.zeros((Nk, d), device=device, dtype=torch.float32)
        v = torch.zeros((Nk, d), device=device, dtype=torch.float32)
        if kind == "count":
            k.normal_(generator=torch.Generator(device=device).manual_seed(7 + g))
            v[:, :PROBE_BITS] = 1.0
        else:
            r = torch.as_tensor(probe_key_order(g if rotate else 0, Nk), device=device)
            k[:, 0] = ((r // 4096) % 64).float()
            k[:, 1] = ((r // 64) % 64).float()
            k[:, 2] = (r % 64).float()
            for bit in range(PROBE_BITS):
                v[:, bit] = ((j >> bit) & 1).float()
        v[:, PROBE_BITS] = float(g + 1)
        ks.append(k)
        vs.append(v)
    qq = q.to(dtype).expand(B, H, Nq, d).contiguous()
    kk = torch.stack(ks).to(dtype).expand(B, Hkv, Nk, d).contiguous()
    vv = torch.stack(vs).to(dtype).expand(B, Hkv, Nk, d).contiguous()
    return qq, kk, vv


# Rising scores: the worst case of the forward's fast pass, which fixes each
# row's reference at its maximum over the first key tile. Q = N(0, 1) + 1 and
# K = N(0, 1) + ramp(j) with the same ramp on every component of key j, so
# every row's scores climb by about `slope` (log2 units) per 64 keys; with
# slope 16 each query block's scores pass its first-tile maximum by more
# than 2^40 within its first four tiles, and again every few tiles after
# each rise of the reference, so the fast pass's bound fails in every block.
RISING_WORKLOADS = {
    "rising": dict(name="fwd_causal_bf16_b8h32n16384d128_rising16", B=8, H=32, N=16384, d=128, dtype="bf16",
                   causal=True, seed=3851, slope=16.0),
}


def make_rising_inputs(cfg, device, shape=None):
    """Seeded bf16 (q, k, v) of the rising-score recipe above, [B, H, N, d]."""
    B, H, N, d = shape or (cfg["B"], cfg["H"], cfg["N"], cfg["d"])
    scale = 1.0 / float(np.sqrt(d))
    step = cfg["slope"] / (scale * float(np.log2(np.e)) * d)  # per 64 keys, on every component of k
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg["seed"])
    q = _randn((B, H, N, d), gen, device).add_(1.0).to(torch.bfloat16)
    ramp = (torch.arange(N, device=device, dtype=torch.float32) / 64 * step).view(1, 1, N, 1)
    k = _randn((B, H, N, d), gen, device).add_(ramp).to(torch.bfloat16)
    v = _randn((B, H, N, d), gen, device).to(torch.bfloat16)
    return q.contiguous(), k.contiguous(), v.contiguous()
