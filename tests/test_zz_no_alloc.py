"""fa_decode_noalloc, the decode entry point that allocates nothing (its
partials live in the library's static per-device scratch), called through
the C ABI with ctypes: two calls in a row, the second on a smaller input,
each compared with fa_decode on the same inputs (the same kernels, so the
results must agree bit for bit, which is within every tolerance of
tests/parity.py) and the first also with the fp64 oracle. The calls must not
change the device memory torch has allocated or reserved. Sizes beyond the
scratch are rejected before any HIP call."""

import ctypes
import math

import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import DECODE_SCRATCH_BYTES, _lib, decode, decode_workspace_bytes
from tests.parity import BF16_ATOL, BF16_RTOL, LSE_ATOL, assert_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H, Hkv, Nq, Nk, d, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    return r(B, H, Nq, d), r(B, Hkv, Nk, d), r(B, Hkv, Nk, d)


def _noalloc(q, k, v, o, lse, causal, scale):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _lib.lib().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        B, H, Hkv, Nq, Nk, d, int(causal), ctypes.c_float(scale), stream)


def test_noalloc_decode_matches_decode_twice_smaller_second():
    shapes = [(8, 32, 8, 1, 16384, 128, True, 6100), (2, 8, 2, 3, 4133, 64, False, 6101)]
    firsts = []
    for i, (B, H, Hkv, Nq, Nk, d, causal, seed) in enumerate(shapes):
        print("[case] noalloc", B, H, Hkv, Nq, Nk, d, causal, flush=True)
        assert decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) <= DECODE_SCRATCH_BYTES
        q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed)
        scale = 1 / math.sqrt(d)
        o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        alloc0, reserved0 = torch.cuda.memory_allocated(), torch.cuda.memory_reserved()
        rc = _noalloc(q, k, v, o, lse, causal, scale)
        assert rc == 0, _lib.status_string(rc)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == alloc0 and torch.cuda.memory_reserved() == reserved0
        o_ref, lse_ref = decode(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"call {i}: differs from fa_decode"
        if i == 0:
            for b in (0, B - 1):
                oo, ll = oracle.forward_decode_heads(host(q[b]), host(k[b]), host(v[b]), scale, causal)
                assert_close(host(o[b]), oo, BF16_ATOL, BF16_RTOL, f"o batch {b}")
                assert_close(host(lse[b]), ll, LSE_ATOL, 0.0, f"lse batch {b}")
            firsts.append((q, k, v, o.clone(), lse.clone(), causal, scale))
    # the first problem again, after the smaller one overwrote the scratch
    q, k, v, o1, l1, causal, scale = firsts[0]
    o = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    assert _noalloc(q, k, v, o, lse, causal, scale) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)


def test_noalloc_decode_rejects_sizes_beyond_the_scratch():
    # B8 H32 Hkv32 Nq1 with a 200K-token cache needs more than the scratch
    B, H, Hkv, Nq, Nk, d = 8, 32, 32, 4, 200000, 128
    assert decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) > DECODE_SCRATCH_BYTES
    A = 1 << 12  # aligned dummy addresses: the call must return before touching them
    rc = _lib.lib().fa_decode_noalloc(A, A, A, A, A, B, H, Hkv, Nq, Nk, d, 1, ctypes.c_float(0.1), None)
    assert rc == _lib.status_codes()["FA_ERR_SCRATCH"]
