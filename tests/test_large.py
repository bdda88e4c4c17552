"""Tensors past 4 GiB, so that element and byte offsets of the later heads
pass 2^31 and 2^32. The bf16 and fp8 forwards and the backward compute every
head independently in a fixed order, so a head's outputs must equal, bit for
bit, those of a call that holds that head alone (whose kernels address it
from offset 0; such calls are checked against the oracle elsewhere). The
decode splits its key range by the size of the whole problem, so its heads
are checked against the oracle instead. Heads checked: the first, the one
whose elements start at 2^31, and the last."""

import math

import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import backward, decode, forward, forward_fp8
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import BF16_ATOL, BF16_RTOL, LSE_ATOL, assert_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_heads_past_4_gib_match_single_head_calls():
    B, H, N, d = 36, 32, 16384, 128
    print("[case] large", B, H, N, d, flush=True)
    assert B * H * N * d * 2 > 2 ** 32
    q, k, v, do = W.make_inputs(dict(dtype="bf16", seed=8100), DEV, with_do=True, shape=(B, H, N, d))
    scale = d ** -0.5
    o, lse = forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    straddle = (2 ** 31) // (N * d)  # the head whose elements cross 2^31
    for b, h in [(0, 0), divmod(straddle, H), (B - 1, H - 1)]:
        one = lambda t: t[b:b + 1, h:h + 1].contiguous()
        o1, lse1 = forward(one(q), one(k), one(v), causal=True, scale=scale)
        dq1, dk1, dv1 = backward(one(q), one(k), one(v), o1, one(do), lse1, causal=True, scale=scale)
        torch.cuda.synchronize()
        for name, big, small in (("o", o, o1), ("lse", lse, lse1), ("dq", dq, dq1), ("dk", dk, dk1),
                                 ("dv", dv, dv1)):
            part = big[b:b + 1, h:h + 1]
            assert torch.equal(part, small), f"{name} of head {(b, h)} differs from the single-head call"
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_fp8_heads_past_4_gib_match_single_head_calls():
    B, H, N, d = 72, 32, 16384, 128
    print("[case] large fp8", B, H, N, d, flush=True)
    assert B * H * N * d > 2 ** 32
    (q, k, v), f = W.make_fp8_inputs(dict(seed=8200), DEV, shape=(B, H, N, d))
    o, lse = forward_fp8(q, k, v, *f, causal=True)
    torch.cuda.synchronize()
    straddle = (2 ** 31) // (N * d)
    for b, h in [(0, 0), divmod(straddle, H), (B - 1, H - 1)]:
        one = lambda t: t[b:b + 1, h:h + 1].contiguous()
        o1, lse1 = forward_fp8(one(q), one(k), one(v), *f, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[b:b + 1, h:h + 1], o1), f"o of head {(b, h)} differs from the single-head call"
        assert torch.equal(lse[b:b + 1, h:h + 1], lse1), f"lse of head {(b, h)} differs from the single-head call"
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_decode_cache_past_4_gib():
    cfg = dict(B=5, H=32, Hkv=32, Nq=2, Nk=131072, d=128, causal=True, seed=8300)
    print("[case] large decode", cfg, flush=True)
    assert cfg["B"] * cfg["Hkv"] * cfg["Nk"] * cfg["d"] * 2 > 2 ** 32
    q, k, v = W.make_decode_inputs(cfg, DEV)
    scale = 1 / math.sqrt(cfg["d"])
    o, lse = decode(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    straddle = (2 ** 31) // (cfg["Nk"] * cfg["d"])
    for b, h in [(0, 0), divmod(straddle, cfg["H"]), (cfg["B"] - 1, cfg["H"] - 1)]:
        o_ref, lse_ref = oracle.forward_decode(host(q[b, h]), host(k[b, h]), host(v[b, h]), scale, True)
        assert_close(host(o[b, h]), o_ref, BF16_ATOL, BF16_RTOL, f"o head {(b, h)}")
        assert_close(host(lse[b, h]), lse_ref, LSE_ATOL, 0.0, f"lse head {(b, h)}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()
