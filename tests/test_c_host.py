"""The C ABI without Python in the loop: tests/c_host/fa_host_check.c, a
plain C program built against include/fa.h and libfa.so (by
__graft_entry__.build()), allocates its own device memory and stream, runs
fa_forward_gqa and writes O and lse; they are compared with the fp64 oracle
(bf16 rule of tests/parity.py). Inputs come from the shared seeded
generator and reach the program through a binary file."""

import math
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import BF16_ATOL, BF16_RTOL, LSE_ATOL, assert_close

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_host", "_build", "fa_host_check")


def _exe(required=True):
    if not os.path.exists(EXE):
        msg = f"{EXE} is missing: run __graft_entry__.build() first"
        pytest.fail(msg) if required else pytest.skip(msg)
    return EXE


def test_host_program_usage_without_gpu():
    """Without its two file arguments the program exits with its usage line
    before it makes any HIP call."""
    r = subprocess.run([_exe(required=False)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def _bits(t):
    return t.view(torch.int16).numpy().astype(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(2, 4, 2, 300, 64, 1), (1, 2, 2, 129, 128, 0), (1, 3, 1, 1, 128, 1)])
def test_host_program_matches_oracle(tmp_path, B, H, Hkv, N, d, causal):
    print("[case] c host", B, H, Hkv, N, d, causal, flush=True)
    q, k, v = W.make_inputs(dict(dtype="bf16", seed=7700 + N + d), "cpu", shape=(B, H, N, d), kv_heads=Hkv)
    scale = 1 / math.sqrt(d)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<6if", B, H, Hkv, N, d, causal, scale))
        for t in (q, k, v):
            f.write(_bits(t).tobytes())
    r = subprocess.run([_exe(), str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    n_o = B * H * N * d * 2
    o_bits = raw[:n_o].view(np.uint16).reshape(B, H, N, d)
    o = torch.from_numpy(o_bits.astype(np.int16)).view(torch.bfloat16).float().numpy()
    lse = raw[n_o:].view(np.float32).reshape(B, H, N)
    g = H // Hkv
    f64 = lambda t: t.float().numpy().astype(np.float64)
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = oracle.forward(f64(q[b, h]), f64(k[b, h // g]), f64(v[b, h // g]), scale, bool(causal))
            assert_close(o[b, h], o_ref, BF16_ATOL, BF16_RTOL, f"o head {(b, h)}")
            assert_close(lse[b, h], lse_ref, LSE_ATOL, 0.0, f"lse head {(b, h)}")
