"""Pins of the shared-key/value-head oracle (oracle/heads.py), CPU only.

It is pinned against PyTorch's fp64 CPU scaled_dot_product_attention with
enable_gqa (a library routine, not this oracle's arithmetic) and its
autograd, and by the special case of one query head per key/value head,
which must reduce to the single-head oracle. A planted grouping mistake
(query head h reading key/value head h % Hkv) must be caught.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import heads as heads_mod


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, scale, causal, do=None):
    t = lambda x: torch.tensor(x[None], dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    if do is None:
        return o[0].detach().numpy()
    o.backward(torch.tensor(do[None], dtype=torch.float64))
    return tq.grad[0].numpy(), tk.grad[0].numpy(), tv.grad[0].numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (8, 8)])
def test_forward_matches_torch_gqa(H, Hkv, causal):
    rng = np.random.default_rng(H * 10 + Hkv + causal)
    N, d = 37, 16
    q, k, v = _rand(rng, H, N, d), _rand(rng, Hkv, N, d), _rand(rng, Hkv, N, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.forward_heads(q, k, v, scale, causal)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale, causal), rtol=1e-12, atol=1e-12)
    # lse against a direct logsumexp of the grouped scores
    for h in range(H):
        s = scale * q[h] @ k[h // (H // Hkv)].T
        if causal:
            s[np.triu_indices(N, 1)] = -np.inf
        np.testing.assert_allclose(lse[h], torch.logsumexp(torch.tensor(s), dim=1).numpy(), rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3)])
def test_backward_matches_torch_gqa_autograd(H, Hkv, causal):
    rng = np.random.default_rng(100 + H * 10 + Hkv + causal)
    N, d = 23, 8
    q, k, v, do = _rand(rng, H, N, d), _rand(rng, Hkv, N, d), _rand(rng, Hkv, N, d), _rand(rng, H, N, d)
    scale = 0.3
    dq, dk, dv = oracle.backward_heads(q, k, v, do, scale, causal)
    rq, rk, rv = _sdpa(q, k, v, scale, causal, do=do)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_one_query_head_per_kv_head_is_the_single_head_oracle():
    rng = np.random.default_rng(7)
    H, N, d = 3, 19, 8
    q, k, v, do = (_rand(rng, H, N, d) for _ in range(4))
    o, lse = oracle.forward_heads(q, k, v, 0.25, True)
    dq, dk, dv = oracle.backward_heads(q, k, v, do, 0.25, True)
    for h in range(H):
        o1, l1 = oracle.forward(q[h], k[h], v[h], 0.25, True)
        g = oracle.backward(q[h], k[h], v[h], do[h], 0.25, True)
        np.testing.assert_array_equal(o[h], o1)
        np.testing.assert_array_equal(lse[h], l1)
        np.testing.assert_array_equal(dq[h], g[0])
        np.testing.assert_array_equal(dk[h], g[1])
        np.testing.assert_array_equal(dv[h], g[2])


def test_kv_head_mapping_and_validation():
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 6, 6) for h in range(6)] == list(range(6))
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


def test_planted_grouping_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(heads_mod, "kv_head", lambda h, H, Hkv: h % Hkv)
    rng = np.random.default_rng(9)
    H, Hkv, N, d = 4, 2, 11, 8
    q, k, v = _rand(rng, H, N, d), _rand(rng, Hkv, N, d), _rand(rng, Hkv, N, d)
    o, _ = heads_mod.forward_heads(q, k, v, 0.4, False)
    assert not np.allclose(o, _sdpa(q, k, v, 0.4, False), atol=1e-6)
