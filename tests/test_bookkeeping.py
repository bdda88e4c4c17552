"""Bit-exact checks of mask and tile bookkeeping at full configuration sizes.

The probe inputs (exact_tiled_attention_38_amd.workloads.probe_inputs) make
the output of every row a closed form of which keys that row sees, so every
row of every head is checked, bit for bit, with no oracle arithmetic:
  count: O == 1 exactly and rint(exp(lse_i)) == number of visible keys
         (i + 1 when causal, N otherwise);
  max:   the bits of O_i spell the largest visible key (i, or N - 1);
  min:   the bits of O_i spell the smallest visible key (0).
Together they pin the visible set of row i to exactly [0, i] (causal) or
[0, N) — the causal mask, tile skipping and ragged-tail predication.
"""

import numpy as np
import pytest
import torch

from exact_tiled_attention_38_amd import forward, forward_f32
from exact_tiled_attention_38_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    # (B, H, N, d, causal): every configuration's shape, plus ragged extras
    (8, 32, 2048, 128, False),
    (8, 32, 16384, 128, True),
    (1, 8, 100000, 128, True),
    (4, 16, 4096, 128, True),
    (2, 16, 700, 128, True),  # 4 heads per XCD: blocks issued across groups of 4 heads
    (2, 2, 777, 64, True),
    (2, 2, 777, 64, False),
    (1, 3, 1, 128, True),
    (3, 1, 4099, 128, False),
]


def _expected_counts(N, causal, device):
    i = torch.arange(N, device=device, dtype=torch.int64)
    return i + 1 if causal else torch.full_like(i, N)


def _run(kind, B, H, N, d, causal, f32=False):
    dtype = torch.float32 if f32 else torch.bfloat16
    q, k, v = W.probe_inputs(kind, B, H, N, d, DEV, dtype=dtype)
    fn = forward_f32 if f32 else forward
    o, lse = fn(q, k, v, causal=causal, scale=W.probe_scale(kind, d))
    torch.cuda.synchronize()
    del q, k, v
    return o, lse


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_count_probe(B, H, N, d, causal):
    print("[case] count", B, H, N, d, causal, flush=True)
    o, lse = _run("count", B, H, N, d, causal)
    assert torch.all(o.float() == 1.0)
    counts = torch.round(torch.exp(lse.double())).to(torch.int64)
    assert torch.equal(counts, _expected_counts(N, causal, DEV).expand(B, H, N))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_max_index_probe(B, H, N, d, causal):
    print("[case] max", B, H, N, d, causal, flush=True)
    o, _ = _run("max", B, H, N, d, causal)
    # each spelled bit is 1 or 0 up to the weight of the runner-up keys: the key one
    # below the largest has softmax weight e^-32 (about 1.3e-14), so a 0 bit may read
    # as such a tiny value, never as anything near 1/2
    bits = o[..., : W.PROBE_BITS].float()
    assert torch.all((bits.abs() < 1 / 64) | ((bits - 1).abs() < 1 / 64))
    idx = W.decode_probe_index(o)
    want = torch.arange(N, device=DEV) if causal else torch.full((N,), N - 1, device=DEV)
    assert torch.equal(idx, want.expand(B, H, N))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_min_index_probe(B, H, N, d, causal):
    print("[case] min", B, H, N, d, causal, flush=True)
    o, _ = _run("min", B, H, N, d, causal)
    idx = W.decode_probe_index(o)
    assert torch.all(idx == 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("N,d", [(256, 64), (129, 128), (1000, 64)])
def test_probes_fp32_path(kind, N, d, causal):
    print("[case] f32", kind, N, d, causal, flush=True)
    o, lse = _run(kind, 1, 2, N, d, causal, f32=True)
    if kind == "count":
        assert torch.all(o == 1.0)
        counts = torch.round(torch.exp(lse.double())).to(torch.int64)
        assert torch.equal(counts, _expected_counts(N, causal, DEV).expand(1, 2, N))
    else:
        idx = W.decode_probe_index(o)
        if kind == "min":
            assert torch.all(idx == 0)
        else:
            want = torch.arange(N, device=DEV) if causal else torch.full((N,), N - 1, device=DEV)
            assert torch.equal(idx, want.expand(1, 2, N))
