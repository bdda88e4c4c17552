"""GPU parity of shared key/value heads (fa_forward_gqa, fa_backward_gqa)
against the fp64 oracle (oracle/heads.py).

Query head h reads key/value head h // (H // Hkv). The forward must match the
oracle to the bf16 tolerance of tests/parity.py, and be bitwise equal to the
multi-head forward run on K and V with each key/value head repeated for its
group (the same kernel reading the same values). The backward must match the
oracle's group-summed dk, dv and per-head dq to the gradient tolerance, and
dq must be bitwise equal to the multi-head dq on repeated K and V.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import _lib, backward, backward_workspace_bytes, forward
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import (BF16_ATOL, BF16_RTOL, GRAD_ATOL, GRAD_RTOL, LSE_ATOL, assert_close,
                          host)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, H, Hkv, N, d, seed, with_do=False):
    return W.make_inputs(dict(dtype="bf16", seed=seed), DEV, with_do=with_do, shape=(B, H, N, d),
                         kv_heads=Hkv)


def _repeat(x, group):
    return x.repeat_interleave(group, dim=1).contiguous()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3)])
@pytest.mark.parametrize("N", [1, 65, 300])
def test_forward_small_shapes(N, H, Hkv, d, causal):
    _say("gqa fwd", N, H, Hkv, d, causal)
    B = 2
    q, k, v = _inputs(B, H, Hkv, N, d, 900 + N + 7 * H + Hkv + d)
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, lse_ref = oracle.forward_heads(host(q[b]), host(k[b]), host(v[b]), scale, causal)
        assert_close(host(o[b]), o_ref, BF16_ATOL, BF16_RTOL, f"o batch {b}")
        assert_close(host(lse[b]), lse_ref, LSE_ATOL, 0.0, f"lse batch {b}")
    # same kernel on repeated key/value heads: bitwise the same result
    o_rep, lse_rep = forward(q, _repeat(k, H // Hkv), _repeat(v, H // Hkv), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_rep) and torch.equal(lse, lse_rep)


@pytest.mark.parametrize("B,H,Hkv,N", [(2, 16, 4, 700), (4, 16, 1, 300), (4, 16, 8, 700)])
def test_causal_heads_interleaved_on_each_xcd(B, H, Hkv, N):
    """32 or 64 query heads of 256-row blocks: each XCD's share of the grid
    is 4 or 8 whole heads, which the causal forward and dQ kernels issue
    longest block first across groups of 4 heads; with 32 key/value heads
    (4, 16, 8, 700) the dK/dV kernel does the same with its key blocks.
    Every head of the forward and of the gradients is checked against the
    oracle."""
    _say("gqa interleaved heads", B, H, Hkv, N)
    d = 128
    q, k, v, do = _inputs(B, H, Hkv, N, d, 2900 + N + Hkv, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, lse_ref = oracle.forward_heads(host(q[b]), host(k[b]), host(v[b]), scale, True)
        assert_close(host(o[b]), o_ref, BF16_ATOL, BF16_RTOL, f"o batch {b}")
        assert_close(host(lse[b]), lse_ref, LSE_ATOL, 0.0, f"lse batch {b}")
        dq_ref, dk_ref, dv_ref = oracle.backward_heads(host(q[b]), host(k[b]), host(v[b]), host(do[b]),
                                                       scale, True)[:3]
        assert_close(host(dq[b]), dq_ref, GRAD_ATOL, GRAD_RTOL, f"dq batch {b}")
        assert_close(host(dk[b]), dk_ref, GRAD_ATOL, GRAD_RTOL, f"dk batch {b}")
        assert_close(host(dv[b]), dv_ref, GRAD_ATOL, GRAD_RTOL, f"dv batch {b}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3)])
@pytest.mark.parametrize("N", [1, 65, 257])
def test_backward_small_shapes(N, H, Hkv, d, causal):
    _say("gqa bwd", N, H, Hkv, d, causal)
    B = 2
    q, k, v, do = _inputs(B, H, Hkv, N, d, 1900 + N + 7 * H + Hkv + d, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    for b in range(B):
        dq_ref, dk_ref, dv_ref = oracle.backward_heads(host(q[b]), host(k[b]), host(v[b]), host(do[b]),
                                                       scale, causal)
        assert_close(host(dv[b]), dv_ref, GRAD_ATOL, GRAD_RTOL, f"dv batch {b}")
        assert_close(host(dk[b]), dk_ref, GRAD_ATOL, GRAD_RTOL, f"dk batch {b}")
        assert_close(host(dq[b]), dq_ref, GRAD_ATOL, GRAD_RTOL, f"dq batch {b}")
    # dq reads K/V exactly as the multi-head dq does on repeated heads
    g = H // Hkv
    dq_rep, _, _ = backward(q, _repeat(k, g), _repeat(v, g), o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_rep)


def test_gqa_entry_points_with_one_query_head_per_kv_head_are_the_plain_ones():
    _say("gqa Hkv == H through the C ABI")
    B, H, N, d = 2, 3, 200, 128
    q, k, v, do = _inputs(B, H, H, N, d, 77, with_do=True)
    scale = 1 / math.sqrt(d)
    L = _lib.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for fwd_name, bwd_name, heads in (("fa_forward", "fa_backward", [B, H]),
                                      ("fa_forward_gqa", "fa_backward_gqa", [B, H, H])):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        rc = getattr(L, fwd_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  *heads, N, d, 1, scale, s)
        assert rc == 0, _lib.status_string(rc)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=DEV)
        rc = getattr(L, bwd_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                  *heads, N, d, 1, scale, s)
        assert rc == 0, _lib.status_string(rc)
        torch.cuda.synchronize()
        outs.append((o, lse, dq, dk, dv))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_binding_rejects_heads_that_do_not_divide():
    q = torch.zeros(1, 6, 16, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="divide"):
        forward(q, k, k)


@pytest.mark.parametrize("kind", ["gqa", "mqa"])
def test_full_size_forward_sampled_rows(kind):
    """B8 H32 N16384 d128 causal with 8 (or 1) key/value heads: sampled rows
    of sampled heads against the oracle, row by row."""
    cfg = W.GQA_WORKLOADS[kind]
    _say("gqa full size", cfg["name"])
    q, k, v = W.make_inputs(cfg, DEV)
    scale = 1 / math.sqrt(cfg["d"])
    o, lse = forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    g = cfg["H"] // cfg["Hkv"]
    rows = W.sample_rows(cfg["N"], 48, cfg["seed"] + 1)
    for b, h in W.sample_heads(cfg["B"], cfg["H"], 3, cfg["seed"] + 2):
        o_ref, lse_ref = oracle.forward(host(q[b, h]), host(k[b, h // g]), host(v[b, h // g]), scale, True,
                                        rows=rows)
        assert_close(host(o[b, h, rows]), o_ref, BF16_ATOL, BF16_RTOL, f"o head {(b, h)}")
        assert_close(host(lse[b, h, rows]), lse_ref, LSE_ATOL, 0.0, f"lse head {(b, h)}")


def test_mid_size_backward_one_kv_head():
    """B1 H8 Hkv2 N4096 d128 causal: every gradient of key/value head 1 and
    of its four query heads against the oracle."""
    _say("gqa bwd mid size")
    B, H, Hkv, N, d = 1, 8, 2, 4096, 128
    q, k, v, do = _inputs(B, H, Hkv, N, d, 3821, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    heads = slice(4, 8)
    dq_ref, dk_ref, dv_ref = oracle.backward_heads(host(q[0, heads]), host(k[0, 1:2]), host(v[0, 1:2]),
                                                   host(do[0, heads]), scale, True)
    assert_close(host(dv[0, 1:2]), dv_ref, GRAD_ATOL, GRAD_RTOL, "dv")
    assert_close(host(dk[0, 1:2]), dk_ref, GRAD_ATOL, GRAD_RTOL, "dk")
    assert_close(host(dq[0, heads]), dq_ref, GRAD_ATOL, GRAD_RTOL, "dq")


def test_backward_deterministic():
    _say("gqa bwd determinism")
    B, H, Hkv, N, d = 2, 8, 2, 1000, 128
    q, k, v, do = _inputs(B, H, Hkv, N, d, 3822, with_do=True)
    o, lse = forward(q, k, v, causal=True)
    first = backward(q, k, v, o, do, lse, causal=True)
    for _ in range(3):
        again = backward(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def _sweep_shapes(count, seed):
    """Seeded random (B, H, Hkv, N, d, causal): head counts that put 1 to 8
    whole heads (or fractions of heads) on each XCD, ragged and tiny N."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        H = Hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.choice([1, 2, 3, 4]))
        N = int(rng.choice([1, 33, 255, 256, 257, 511, 700, 1024, 1500, 2049]))
        d = int(rng.choice([64, 128]))
        out.append((B, H, Hkv, N, d, bool(rng.integers(2))))
    return out


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", _sweep_shapes(48, 3838))
def test_random_shapes_forward_and_backward(B, H, Hkv, N, d, causal):
    """A seeded sweep over grid sizes, head sharing, ragged lengths and both
    masks: every head's O, lse and gradients against the oracle."""
    _say("sweep", B, H, Hkv, N, d, causal)
    q, k, v, do = _inputs(B, H, Hkv, N, d, 4100 + N + 3 * H + Hkv + d + B, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, lse_ref = oracle.forward_heads(host(q[b]), host(k[b]), host(v[b]), scale, causal)
        assert_close(host(o[b]), o_ref, BF16_ATOL, BF16_RTOL, f"o batch {b}")
        assert_close(host(lse[b]), lse_ref, LSE_ATOL, 0.0, f"lse batch {b}")
        dq_ref, dk_ref, dv_ref = oracle.backward_heads(host(q[b]), host(k[b]), host(v[b]), host(do[b]),
                                                       scale, causal)[:3]
        assert_close(host(dq[b]), dq_ref, GRAD_ATOL, GRAD_RTOL, f"dq batch {b}")
        assert_close(host(dk[b]), dk_ref, GRAD_ATOL, GRAD_RTOL, f"dk batch {b}")
        assert_close(host(dv[b]), dv_ref, GRAD_ATOL, GRAD_RTOL, f"dv batch {b}")
