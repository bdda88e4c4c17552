"""Bit-exact bookkeeping probes for the rows built beyond the dense forward:
decode with its key splits, the block-sparse key-block lists, and shared
key/value heads. As in test_bookkeeping.py, the probe inputs
(workloads.probe_heads_inputs) make every output a closed form of which keys
a row sees (tests/probes.py, itself checked against the fp64 oracle in
tests/test_probe_expectations.py), so every row is compared bit for bit:

  count: Q = 0 and V = 1, so P = 1 on every visible key: the first
         PROBE_BITS columns of O are exactly 1 and rint(exp(lse_i)) is the
         number of visible keys. A key dropped or counted twice at a split
         boundary, a list edge or a tile edge changes that integer.
  max:   s_ij = 32 r_g(j) exactly (r_g a per-K/V-head rotation of the key
         order), so O_i spells the visible key j that maximises r_g(j);
  min:   the same for the minimum.
  head:  column PROBE_BITS of V holds g + 1 for key/value head g, so query
         head h must read h // (H / Hkv) + 1 there (exactly with the count
         probe; rounded to the nearest integer otherwise, as the key bits
         are); with the rotation the spelled key also depends on which K
         head was read.
Rows that see no key (block-sparse only) must give O = 0 and lse = -inf.
"""

import numpy as np
import pytest
import torch

from exact_tiled_attention_38_amd import SPARSE_BLOCK_M as BM
from exact_tiled_attention_38_amd import SPARSE_BLOCK_N as BN
from exact_tiled_attention_38_amd import decode, forward, forward_block_sparse
from exact_tiled_attention_38_amd import workloads as W
from tests import probes as P

pytestmark = pytest.mark.gpu
DEV = "cuda"
PB = W.PROBE_BITS


def _say(*a):
    print("[case]", *a, flush=True)


def _check(kind, o, lse, want_count, want_index, mark):
    """o [B, H, R, d], lse [B, H, R]; want_count / want_index int64 numpy [H, R];
    mark float [H], the head marker every seen row of head h must read."""
    B, H, R, _ = o.shape
    seen = torch.as_tensor(want_count > 0, device=DEV).expand(B, H, R)
    m = torch.as_tensor(mark, dtype=torch.float32, device=DEV).view(1, H, 1).expand(B, H, R)
    col = o[..., PB].float()[seen]
    # (the marker is g + 1 times the ratio of the bf16-rounded P sum to the fp32
    # one, which is 1 within 2^-8, so it reads g + 1 to within (g + 1) / 256
    # and rounds to it exactly; with the count probe's P = 1 it is exact)
    assert torch.all((col - m[seen]).abs() <= m[seen] / 64), f"{kind}: head marker column"
    assert torch.equal(torch.round(col), m[seen]), f"{kind}: head marker column"
    if (~seen).any():
        assert torch.all(o[~seen].float() == 0) and torch.all(lse[~seen] == -float("inf")), f"{kind}: unseen rows"
    if kind == "count":
        assert torch.all(o[..., :PB][seen].float() == 1.0), "count: O != 1"
        counts = torch.round(torch.exp(lse.double())).to(torch.int64)
        want = torch.as_tensor(want_count, device=DEV).expand(B, H, R)
        bad = int((counts[seen] != want[seen]).sum())
        assert bad == 0, f"count: {bad} rows differ"
    else:
        bits = o[..., :PB].float()[seen]
        assert torch.all((bits.abs() < 1 / 64) | ((bits - 1).abs() < 1 / 64)), f"{kind}: bits not 0/1"
        idx = W.decode_probe_index(o)
        want = torch.as_tensor(want_index, device=DEV).expand(B, H, R)
        bad = int((idx[seen] != want[seen]).sum())
        assert bad == 0, f"{kind}: {bad} rows differ"


def _marks(H, Hkv):
    return np.arange(H) // (H // Hkv) + 1.0


# ---------------------------------------------------------------- decode

DECODE_SHAPES = [
    # (B, H, Hkv, Nq, Nk, d, causal): the three decode workloads, then caches
    # whose key splits end at varied offsets, with shared heads and Nq > 1
    (8, 32, 32, 1, 16384, 128, True),
    (8, 32, 8, 1, 16384, 128, True),
    (1, 8, 8, 1, 100000, 128, True),
    (2, 8, 2, 3, 1000, 128, True),
    (2, 8, 2, 3, 1000, 64, False),
    (2, 8, 1, 5, 4133, 128, True),
    (1, 6, 3, 2, 4133, 64, False),
    (1, 8, 2, 1, 100000, 128, False),
    (1, 4, 4, 40, 100000, 64, True),
]


@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", DECODE_SHAPES)
def test_decode_probes(kind, B, H, Hkv, Nq, Nk, d, causal):
    _say("decode probe", kind, B, H, Hkv, Nq, Nk, d, causal)
    q, k, v = W.probe_heads_inputs(kind, B, H, Hkv, Nq, Nk, d, DEV)
    o, lse = decode(q, k, v, causal=causal, scale=W.probe_scale(kind, d))
    torch.cuda.synchronize()
    count, index = P.dense_expected(kind, H, Hkv, Nq, Nk, causal)
    _check(kind, o, lse, count, index, _marks(H, Hkv))


# ---------------------------------------------------------------- shared heads, forward

GQA_SHAPES = [
    (8, 32, 8, 16384, 128, True),   # the shared-head workload
    (8, 32, 1, 16384, 128, True),   # the multi-query workload
    (2, 6, 3, 777, 64, True),
    (2, 6, 3, 777, 128, False),
    (1, 8, 2, 4099, 128, True),
]


@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("B,H,Hkv,N,d,causal", GQA_SHAPES)
def test_shared_head_forward_probes(kind, B, H, Hkv, N, d, causal):
    _say("gqa probe", kind, B, H, Hkv, N, d, causal)
    q, k, v = W.probe_heads_inputs(kind, B, H, Hkv, N, N, d, DEV)
    o, lse = forward(q, k, v, causal=causal, scale=W.probe_scale(kind, d))
    torch.cuda.synchronize()
    count, index = P.dense_expected(kind, H, Hkv, N, N, causal)
    _check(kind, o, lse, count, index, _marks(H, Hkv))


# ---------------------------------------------------------------- block-sparse lists

SPARSE_CASES = [
    # (B, H, Hkv, N, d, causal, selection): the block-sparse workload's own
    # lists, then shuffled random lists with empty rows, ragged N, both masks,
    # and shared heads
    (8, 32, 32, 16384, 128, True, "workload"),
    (2, 4, 4, 4133, 128, True, "random"),
    (2, 4, 2, 4133, 64, False, "random"),
    (1, 3, 1, 777, 128, True, "random"),
]


@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("B,H,Hkv,N,d,causal,selection", SPARSE_CASES)
def test_block_sparse_probes(kind, B, H, Hkv, N, d, causal, selection):
    _say("sparse probe", kind, B, H, Hkv, N, d, causal, selection)
    if selection == "workload":
        cfg = W.SPARSE_WORKLOADS["sparse"]
        row_ptr, cols = W.sparse_selection(B, H, N, cfg["seed"], cfg["keep"])
    else:
        rng = np.random.default_rng(5000 + N + d + causal)
        row_ptr, cols = P.random_lists(rng, B * H * -(-N // BM), -(-N // BN), 0.3, 7)
    q, k, v = W.probe_heads_inputs(kind, B, H, Hkv, N, N, d, DEV, rotate=False)
    o, lse = forward_block_sparse(q, k, v, torch.as_tensor(row_ptr, device=DEV),
                                  torch.as_tensor(cols, device=DEV), causal=causal,
                                  scale=W.probe_scale(kind, d))
    torch.cuda.synchronize()
    count, index = P.sparse_expected(kind, N, row_ptr, cols, causal, B * H)
    # lists are per (b, h): check as B * H heads of one batch
    marks = np.tile(_marks(H, Hkv), B)
    _check(kind, o.view(1, B * H, N, d), lse.view(1, B * H, N), count, index, marks)
