"""GPU parity of the forward path (fa_forward, fa_forward_f32) against the fp64 oracle.

Every configuration is checked on the same seeded inputs the GPU consumed,
read back exactly. Where the oracle cannot afford every row, it checks a
seeded sample of whole heads and of rows in every head; the bookkeeping
probes (test_bookkeeping.py) cover every row at full size.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import forward, forward_f32
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import BF16_ATOL, BF16_RTOL, F32_ATOL, LSE_ATOL, assert_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _check_heads(q, k, v, o, lse, scale, causal, heads, rows=None, f32=False):
    """Compare O and lse of the given (b, h) heads (all rows or `rows`) with the oracle."""
    for b, h in heads:
        qh, kh, vh = host(q[b, h]), host(k[b, h]), host(v[b, h])
        o_ref, lse_ref = oracle.forward(qh, kh, vh, scale, causal, rows=rows)
        sel = slice(None) if rows is None else torch.as_tensor(rows)
        og, lg = host(o[b, h][sel]), host(lse[b, h][sel])
        if f32:
            assert_close(og, o_ref, F32_ATOL, 0.0, f"O head {(b, h)}")
            assert_close(lg, lse_ref, F32_ATOL, 0.0, f"lse head {(b, h)}")
        else:
            assert_close(og, o_ref, BF16_ATOL, BF16_RTOL, f"O head {(b, h)}")
            assert_close(lg, lse_ref, LSE_ATOL, 0.0, f"lse head {(b, h)}")


# ---------------------------------------------------------------- configuration 1 (fp32)


def test_config1_fp32_exact():
    cfg = W.config(1)
    _say("config 1", cfg["name"])
    q, k, v = W.make_inputs(cfg, DEV)
    o, lse = forward_f32(q, k, v, causal=cfg["causal"], scale=cfg["scale"])
    torch.cuda.synchronize()
    _check_heads(q, k, v, o, lse, cfg["scale"], cfg["causal"], [(0, 0)], f32=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 129, 300])
def test_fp32_small_shapes(N, d, causal):
    _say("f32 sweep", N, d, causal)
    cfg = dict(dtype="f32", seed=11 + N + d)
    q, k, v = W.make_inputs(cfg, DEV, shape=(2, 2, N, d))
    scale = 1 / math.sqrt(d)
    o, lse = forward_f32(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check_heads(q, k, v, o, lse, scale, causal, [(0, 0), (1, 1)], f32=True)


# ---------------------------------------------------------------- small bf16 shapes, all rows


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 17, 31, 32, 33, 63, 64, 65, 127, 129, 255, 256, 257, 300, 511, 777])
def test_bf16_small_shapes_all_rows(N, d, causal):
    _say("bf16 sweep", N, d, causal)
    cfg = dict(dtype="bf16", seed=1000 + N * 7 + d, q_mult=4.0 if N % 2 else 1.0)
    B, H = 2, 3
    q, k, v = W.make_inputs(cfg, DEV, shape=(B, H, N, d))
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check_heads(q, k, v, o, lse, scale, causal, [(b, h) for b in range(B) for h in range(H)])


def test_bf16_nondefault_scale():
    _say("bf16 scale 0.37")
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=5), DEV, shape=(1, 2, 200, 128))
    o, lse = forward(q, k, v, causal=True, scale=0.37)
    torch.cuda.synchronize()
    _check_heads(q, k, v, o, lse, 0.37, True, [(0, 0), (0, 1)])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N, v_log2", [(300, 0), (777, 0), (2000, 0), (300, 110), (500, 100)])
def test_bf16_rising_scores_all_rows(N, d, causal, v_log2):
    """Scores that rise along the key index by about 4 (log2 units) per 64
    keys, so the maxima of a row's first keys are far below those of its
    later keys. At N = 300 the later tiles' P reach about 2^19 against the
    first tile's maximum, which the kernel keeps as the reference; from N =
    777 on, a tile's row sums pass 2^40 (at N = 2000 they overflow fp32) and
    the kernel must rerun such blocks with per-tile maxima, while causal
    blocks near the start stay below that bound, so both kinds of block occur
    in one launch. With V scaled by 2^110 at N = 300 the accumulator, not
    the row sum, leaves the fp32 range against the first tile's maximum
    (about 2^135), while with per-tile maxima it stays near 2^122. At N =
    500 with V of about +-2^100 (1e30, random signs) P reaches about 2^35
    against the first tile's maximum, below the row-sum bound, but single
    products reach 2^137: accumulators overflow with both signs and become
    NaN (inf - inf) rather than inf, which the kernel must flag as well; the
    oracle's O is finite. Every row is compared."""
    _say("rising scores", N, d, causal, v_log2)
    g = torch.Generator().manual_seed(77 + N + d)
    B, H = 1, 2
    scale = 1 / math.sqrt(d)
    step = 4.0 / (scale * math.log2(math.e) * d)  # per 64 keys, on every component of k
    ramp = (torch.arange(N, dtype=torch.float32) / 64 * step).view(1, 1, N, 1)
    q = (torch.randn(B, H, N, d, generator=g) + 1.0).to(torch.bfloat16).to(DEV)
    k = (torch.randn(B, H, N, d, generator=g) + ramp).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    # (a power-of-two factor is exact in bf16 and commutes with every
    # rounding, so O / 2^v_log2 is compared with the oracle on the unscaled V)
    o, lse = forward(q, k, v * 2.0**v_log2, causal=causal, scale=scale)
    o2, lse2 = forward(q, k, v * 2.0**v_log2, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    # blocks that rerun are as deterministic as the rest
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    _check_heads(q, k, v, o * 2.0**-v_log2, lse, scale, causal, [(0, 0), (0, 1)])


# ---------------------------------------------------------------- configuration 2


@pytest.fixture(scope="module")
def run_config2():
    cfg = W.config(2)
    _say("config 2", cfg["name"])
    q, k, v = W.make_inputs(cfg, DEV)
    o, lse = forward(q, k, v, causal=cfg["causal"], scale=cfg["scale"])
    torch.cuda.synchronize()
    return cfg, q, k, v, o, lse


@pytest.mark.timeout(900)
def test_config2_all_rows(run_config2):
    cfg, q, k, v, o, lse = run_config2
    heads = [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])]
    _check_heads(q, k, v, o, lse, cfg["scale"], cfg["causal"], heads)


def test_forward_is_deterministic(run_config2):
    cfg, q, k, v, o, lse = run_config2
    for _ in range(5):
        o2, lse2 = forward(q, k, v, causal=cfg["causal"], scale=cfg["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
        assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))


@pytest.mark.parametrize("causal", [True, False])
def test_forward_is_deterministic_ragged(causal):
    # a ragged length (not a multiple of any tile), every output rewritten
    # from a NaN-filled buffer on each run
    _say("determinism ragged", causal)
    B, H, N, d = 2, 3, 1000, 128
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=8), DEV, shape=(B, H, N, d))
    ref = None
    for _ in range(8):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N), float("nan"), device=DEV)
        forward(q, k, v, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert not torch.isnan(o.float()).any() and not torch.isnan(lse).any()
        if ref is None:
            ref = (o.clone(), lse.clone())
            continue
        diff = (o.view(torch.int16) != ref[0].view(torch.int16)).any(-1).nonzero()
        assert diff.shape[0] == 0, f"rows differing between runs: {diff.shape[0]}, first {diff[:6].tolist()}"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32))


# ---------------------------------------------------------------- configuration 3


@pytest.fixture(scope="module")
def run_config3():
    cfg = W.config(3)
    _say("config 3", cfg["name"])
    q, k, v = W.make_inputs(cfg, DEV)
    o, lse = forward(q, k, v, causal=cfg["causal"], scale=cfg["scale"])
    torch.cuda.synchronize()
    yield cfg, q, k, v, o, lse
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_config3_whole_heads(run_config3):
    cfg, q, k, v, o, lse = run_config3
    heads = W.sample_heads(cfg["B"], cfg["H"], 4, cfg["seed"] + 1)
    _check_heads(q, k, v, o, lse, cfg["scale"], cfg["causal"], heads)


@pytest.mark.timeout(900)
def test_config3_rows_of_every_head(run_config3):
    cfg, q, k, v, o, lse = run_config3
    rows = W.sample_rows(cfg["N"], 512, cfg["seed"] + 1)
    heads = [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])]
    _check_heads(q, k, v, o, lse, cfg["scale"], cfg["causal"], heads, rows=rows)


# ---------------------------------------------------------------- configuration 4


@pytest.mark.timeout(900)
def test_config4_rows_and_no_quadratic_allocation():
    cfg = W.config(4)
    _say("config 4", cfg["name"])
    q, k, v = W.make_inputs(cfg, DEV)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    free_before, _ = torch.cuda.mem_get_info()
    forward(q, k, v, causal=True, scale=cfg["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    # nothing beyond the caller's own outputs: no N x N (20 GB per head) buffer, no scratch
    assert torch.cuda.max_memory_allocated() - base_alloc == 0
    assert abs(free_before - free_after) < 8 * 2**20
    rows = W.sample_rows(N, 2048, cfg["seed"] + 1)
    _check_heads(q, k, v, o, lse, cfg["scale"], True, [(0, h) for h in range(H)], rows=rows)


# ---------------------------------------------------------------- output guard bands


def test_outputs_write_nothing_outside_their_bounds():
    _say("guard bands")
    B, H, N, d = 2, 3, 333, 128
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=99), DEV, shape=(B, H, N, d))
    pad = 4096
    n_o, n_l = B * H * N * d, B * H * N
    obuf = torch.full((n_o + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((n_l + 2 * pad,), -7.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + n_o].view(B, H, N, d)
    lse = lbuf[pad:pad + n_l].view(B, H, N)
    forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == -7.0) and torch.all(obuf[pad + n_o:] == -7.0)
    assert torch.all(lbuf[:pad] == -7.0) and torch.all(lbuf[pad + n_l:] == -7.0)
    assert torch.all(torch.isfinite(o.float())) and torch.all(torch.isfinite(lse))


@pytest.mark.parametrize("B,H,N,causal", [(8, 32, 2048, False), (4, 16, 4099, True)])
def test_bf16_many_units_per_workgroup_deterministic(B, H, N, causal):
    """Shapes with more (head, query block) units than compute units, so each
    workgroup runs several units in turn and its waves reuse the LDS ring
    across them: repeated launches must agree bit for bit (a wave reading a
    ring slot that another wave's next load already overwrote would not),
    and one head is checked against the oracle."""
    _say("many units", B, H, N, causal)
    cfg = dict(dtype="bf16", seed=31 + N, q_mult=4.0)
    q, k, v = W.make_inputs(cfg, DEV, shape=(B, H, N, 128))
    scale = 1 / math.sqrt(128)
    first = forward(q, k, v, causal=causal, scale=scale)
    for _ in range(6):
        again = forward(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
    _check_heads(q, k, v, first[0], first[1], scale, causal, [(B - 1, H - 1)])


@pytest.mark.parametrize("B,H,N,d", [(2, 16, 700, 128), (4, 16, 300, 64), (2, 16, 513, 64)])
def test_bf16_causal_heads_interleaved_on_each_xcd(B, H, N, d):
    """32 or 64 heads of 256-row blocks: each XCD's share of the grid is 4 or
    8 whole heads, which the causal forward issues longest block first across
    groups of 4 heads. Every row of every head is checked."""
    _say("interleaved heads", B, H, N, d)
    cfg = dict(dtype="bf16", seed=77 + N + d, q_mult=4.0)
    q, k, v = W.make_inputs(cfg, DEV, shape=(B, H, N, d))
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    _check_heads(q, k, v, o, lse, scale, True, [(b, h) for b in range(B) for h in range(H)])
