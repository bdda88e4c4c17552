"""The closed-form probe expectations (tests/probes.py) against the fp64
oracle on the same probe inputs, on small shapes on the CPU: the oracle's
lse must give the expected key counts, and its O the expected key index and
head marker. This pins the expectation code and the probe construction
independently of the HIP path, before the GPU tests use them at full size."""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import workloads as W
from tests import probes as P

PB = W.PROBE_BITS


def _spelled(o):
    return (np.rint(o[..., :PB]).astype(np.int64) << np.arange(PB)).sum(-1)


def _compare(kind, o, lse, count, index, marks):
    """o [H, R, d], lse [H, R] from the oracle (fp64 numpy)."""
    seen = count > 0
    assert np.all(np.isneginf(lse[~seen])) and np.all(o[~seen] == 0)
    assert np.allclose(o[..., PB][seen], np.broadcast_to(marks[:, None], seen.shape)[seen], rtol=0, atol=1e-9)
    if kind == "count":
        assert np.array_equal(np.rint(np.exp(lse[seen])).astype(np.int64), count[seen])
        assert np.allclose(o[..., :PB][seen], 1.0, rtol=0, atol=1e-12)
    else:
        assert np.array_equal(_spelled(o)[seen], index[seen])


def _host(t):
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("H,Hkv,Nq,Nk,d,causal", [(4, 2, 3, 200, 64, True), (4, 1, 1, 150, 64, False),
                                                  (6, 3, 7, 91, 64, True), (2, 2, 91, 91, 64, True)])
def test_decode_and_shared_head_expectations(kind, H, Hkv, Nq, Nk, d, causal):
    q, k, v = W.probe_heads_inputs(kind, 1, H, Hkv, Nq, Nk, d, "cpu")
    o, lse = oracle.forward_decode_heads(_host(q[0]), _host(k[0]), _host(v[0]), W.probe_scale(kind, d), causal)
    count, index = P.dense_expected(kind, H, Hkv, Nq, Nk, causal)
    _compare(kind, o, lse, count, index, np.arange(H) // (H // Hkv) + 1.0)


@pytest.mark.parametrize("kind", ["count", "max", "min"])
@pytest.mark.parametrize("N,causal,seed", [(300, True, 1), (300, False, 2), (600, True, 3)])
def test_block_sparse_expectations(kind, N, causal, seed):
    H = 2
    n_qb, n_kb = -(-N // P.SPARSE_BM), -(-N // P.SPARSE_BN)
    rng = np.random.default_rng(seed)
    row_ptr, cols = P.random_lists(rng, H * n_qb, n_kb, 0.4, 3)
    q, k, v = W.probe_heads_inputs(kind, 1, H, H, N, N, 64, "cpu", rotate=False)
    count, index = P.sparse_expected(kind, N, row_ptr, cols, causal, H)
    for h in range(H):
        rp = row_ptr[h * n_qb:(h + 1) * n_qb + 1] - row_ptr[h * n_qb]
        cc = cols[row_ptr[h * n_qb]:row_ptr[(h + 1) * n_qb]]
        o, lse = oracle.forward_block_sparse(_host(q[0, h]), _host(k[0, h]), _host(v[0, h]),
                                             W.probe_scale(kind, 64), causal, rp, cc, P.SPARSE_BM, P.SPARSE_BN)
        _compare(kind, o[None], lse[None], count[h:h + 1], index[h:h + 1], np.array([h + 1.0]))


def test_sparse_expectations_catch_a_dropped_block():
    """A list edited by one block must change some expected count (the check is not vacuous)."""
    N, H = 700, 1
    rng = np.random.default_rng(9)
    row_ptr, cols = P.random_lists(rng, 3, 11, 0.5, 0)
    base, _ = P.sparse_expected("count", N, row_ptr, cols, True, H)
    cut = row_ptr.copy()
    cut[1:] -= 1  # drop the first list's first block
    cnt2, _ = P.sparse_expected("count", N, cut, cols[1:], True, H)
    assert not np.array_equal(base, cnt2)
