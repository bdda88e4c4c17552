"""Pins of the block-sparse oracle (oracle/sparse.py), CPU only.

Pinned against PyTorch's fp64 CPU scaled_dot_product_attention with a
boolean mask built here, element by element, from the selection (not by the
oracle's own block_mask), against the dense oracle when every block is
selected (causal and not), by the empty selection (O = 0, lse = -inf), by
the selection of exactly the causal lower block triangle (equals the causal
oracle on rows whose blocks are whole), and by a planted transposition of
the block indices.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import sparse as sparse_mod


def _csr(lists):
    row_ptr = np.cumsum([0] + [len(x) for x in lists]).astype(np.int64)
    cols = np.array([c for x in lists for c in x], dtype=np.int64)
    return row_ptr, cols


def _random_selection(rng, n_qb, n_kb, density):
    return [sorted(rng.choice(n_kb, size=rng.binomial(n_kb, density), replace=False).tolist())
            for _ in range(n_qb)]


def _elementwise_mask(n, lists, bm, bn, causal):
    m = torch.zeros(n, n, dtype=torch.bool)
    for i in range(n):
        for j in range(n):
            if (j // bn) in lists[i // bm] and (not causal or j <= i):
                m[i, j] = True
    return m


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,bm,bn,density", [(37, 8, 4, 0.5), (64, 16, 8, 0.3), (50, 32, 16, 0.7)])
def test_matches_sdpa_with_elementwise_mask(n, bm, bn, density, causal):
    rng = np.random.default_rng(n + bm + bn + causal)
    d = 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lists = _random_selection(rng, -(-n // bm), -(-n // bn), density)
    lists[0] = sorted(set(lists[0]) | {0})  # keep row 0 non-empty under the causal mask
    row_ptr, cols = _csr(lists)
    o, lse = oracle.forward_block_sparse(q, k, v, 0.4, causal, row_ptr, cols, bm, bn)
    mask = _elementwise_mask(n, lists, bm, bn, causal)
    seen = mask.any(1).numpy()
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    ref = F.scaled_dot_product_attention(t(q)[None], t(k)[None], t(v)[None], attn_mask=mask, scale=0.4)[0]
    np.testing.assert_allclose(o[seen], ref.numpy()[seen], rtol=1e-12, atol=1e-12)
    s = 0.4 * t(q) @ t(k).T
    s[~mask] = -math.inf
    np.testing.assert_allclose(lse[seen], torch.logsumexp(s, 1).numpy()[seen], rtol=1e-12)
    assert np.all(o[~seen] == 0) and np.all(lse[~seen] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_every_block_selected_is_dense(causal):
    rng = np.random.default_rng(1)
    n, d, bm, bn = 45, 8, 16, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    n_kb = -(-n // bn)
    row_ptr, cols = _csr([list(range(n_kb))] * -(-n // bm))
    o, lse = oracle.forward_block_sparse(q, k, v, 0.3, causal, row_ptr, cols, bm, bn)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)


def test_empty_selection():
    rng = np.random.default_rng(2)
    n, d = 20, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    row_ptr, cols = _csr([[], [1], []])
    o, lse = oracle.forward_block_sparse(q, k, v, 0.5, False, row_ptr, cols, 8, 8)
    assert np.all(o[:8] == 0) and np.all(lse[:8] == -np.inf)
    assert np.all(o[16:] == 0) and np.all(lse[16:] == -np.inf)
    assert np.all(np.isfinite(lse[8:16]))


def test_lower_block_triangle_with_causal_is_the_causal_oracle():
    rng = np.random.default_rng(3)
    n, d, b = 64, 8, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    row_ptr, cols = _csr([list(range(r + 1)) for r in range(n // b)])
    o, lse = oracle.forward_block_sparse(q, k, v, 0.25, True, row_ptr, cols, b, b)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.25, True)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)


def test_planted_transposition_is_caught(monkeypatch):
    rng = np.random.default_rng(4)
    n, d, bm, bn = 48, 8, 16, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lists = [[0, 3], [1, 2, 5], [0, 4]]
    row_ptr, cols = _csr(lists)
    good, _ = oracle.forward_block_sparse(q, k, v, 0.3, False, row_ptr, cols, bm, bn)
    real = sparse_mod.block_mask
    monkeypatch.setattr(sparse_mod, "block_mask", lambda nn, rp, cc, m_, n_, c: real(nn, rp, cc, m_, n_, c).T)
    bad, _ = sparse_mod.forward_block_sparse(q, k, v, 0.3, False, row_ptr, cols, bm, bn)
    assert not np.allclose(np.nan_to_num(bad), good, atol=1e-6)


def test_row_subset_matches_full():
    rng = np.random.default_rng(6)
    n, d, bm, bn = 70, 8, 16, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lists = _random_selection(rng, -(-n // bm), -(-n // bn), 0.4)
    lists[0] = sorted(set(lists[0]) | {0})
    row_ptr, cols = _csr(lists)
    for causal in (False, True):
        o, lse = oracle.forward_block_sparse(q, k, v, 0.3, causal, row_ptr, cols, bm, bn)
        rows = np.array([0, 5, 16, 33, 69])
        o2, lse2 = oracle.forward_block_sparse(q, k, v, 0.3, causal, row_ptr, cols, bm, bn, rows=rows)
        np.testing.assert_array_equal(o2, o[rows])
        np.testing.assert_array_equal(lse2, lse[rows])
