"""Race check of the bf16 forward's LDS pipeline (the dense, shared-head and
block-sparse instances). libfa_safe.so is libfa.so with the forward built
with FA_SAFE_SYNC=1: every tile load is waited for at each step's end and a
workgroup barrier follows each LDS read phase, so no wave can read a tile
before its load landed or see it overwritten while it still reads it. The
arithmetic is unchanged, so the pipelined forward must give the same bits;
a race would show as a difference (or as run-to-run noise, which the
determinism tests look for)."""

import ctypes
import math
import os

import numpy as np
import pytest
import torch

from exact_tiled_attention_38_amd import _lib
from exact_tiled_attention_38_amd import workloads as W
from tests import probes as P

pytestmark = pytest.mark.gpu
DEV = "cuda"
SAFE = os.path.join(os.path.dirname(_lib.LIB_PATH), "libfa_safe.so")


@pytest.fixture(scope="module")
def libs():
    if not os.path.exists(SAFE):
        pytest.fail("libfa_safe.so is missing: build with exact_tiled_attention_38_amd/csrc/build.py")
    assert open(SAFE, "rb").read() != open(_lib.LIB_PATH, "rb").read()
    safe = ctypes.CDLL(SAFE)
    for name in ("fa_forward_gqa", "fa_forward_block_sparse"):
        fn = getattr(safe, name)
        fn.restype, fn.argtypes = _lib.SIGNATURES[name]
    return _lib.lib(), safe


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _fwd(L, q, k, v, causal, scale, sel=None):
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    if sel is None:
        rc = L.fa_forward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, k.shape[1], N, d, int(causal), scale, _stream())
    else:
        rp, cols = sel
        rc = L.fa_forward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       rp.data_ptr(), cols.data_ptr(), cols.numel(), B, H, k.shape[1], N, d,
                                       int(causal), scale, _stream())
    assert rc == 0, _lib.status_string(rc)
    return o, lse


def _same(libs, q, k, v, causal, scale, sel=None):
    a = _fwd(libs[0], q, k, v, causal, scale, sel)
    b = _fwd(libs[1], q, k, v, causal, scale, sel)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]), "O differs from the race-check build"
    assert torch.equal(a[1], b[1]), "lse differs from the race-check build"


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,q_mult", [
    (2, 4, 4, 4099, 128, True, 1.0),
    (8, 32, 32, 2048, 128, False, 4.0),
    (2, 3, 3, 777, 64, True, 4.0),
    (2, 8, 2, 3000, 128, True, 1.0),
    (1, 2, 2, 100000, 128, True, 1.0),
])
def test_forward_matches_race_check_build(libs, B, H, Hkv, N, d, causal, q_mult):
    print("[case] safe-sync", B, H, Hkv, N, d, causal, q_mult, flush=True)
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=7000 + N + d, q_mult=q_mult), DEV, shape=(B, H, N, d),
                            kv_heads=Hkv)
    _same(libs, q, k, v, causal, 1 / math.sqrt(d))


def test_rerun_blocks_match_race_check_build(libs):
    print("[case] safe-sync rising", flush=True)
    cfg = dict(W.RISING_WORKLOADS["rising"], slope=4.0)
    q, k, v = W.make_rising_inputs(cfg, DEV, shape=(1, 4, 2000, 128))
    _same(libs, q, k, v, True, 1 / math.sqrt(128))


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_matches_race_check_build(libs, causal):
    print("[case] safe-sync sparse", causal, flush=True)
    B, H, N, d = 2, 4, 4133, 128
    rng = np.random.default_rng(7100 + causal)
    rp, cols = P.random_lists(rng, B * H * -(-N // 256), -(-N // 64), 0.3, 7)
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=7101), DEV, shape=(B, H, N, d))
    sel = (torch.as_tensor(rp, device=DEV), torch.as_tensor(cols, device=DEV))
    _same(libs, q, k, v, causal, 1 / math.sqrt(d), sel)
