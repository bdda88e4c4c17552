"""Pins of the decode and merge oracle (oracle/decode.py), CPU only.

forward_decode is pinned against PyTorch's fp64 CPU
scaled_dot_product_attention given an explicit boolean mask built here from
the reading (query i at position Nk - Nq + i sees keys j <= that position),
against torch.logsumexp, and by its special cases (Nq = Nk is the ordinary
causal oracle, Nq = 1 sees every key). merge_partials is pinned by the
worked example of "Online softmax intuition" (blocks [1, 2, 3] and [4]),
whose merged values are the one-shot closed forms, and by the identity that
merging the results over disjoint key sets (empty ones included) gives the
result over all keys. Planted mistakes (a mask off by one, an unweighted
merge) must be caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import decode as decode_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_worked_example.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_masked(q, k, v, scale, causal):
    nq, nk = q.shape[-2], k.shape[-2]
    mask = None
    if causal:
        pos = torch.arange(nk - nq, nk)[:, None]
        mask = torch.arange(nk)[None, :] <= pos
    t = lambda x: torch.tensor(x[None], dtype=torch.float64)
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=scale,
                                       enable_gqa=q.ndim == 3 and q.shape[0] != k.shape[0])
    return o[0].numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 37), (3, 37), (8, 8), (5, 129), (16, 300)])
def test_decode_matches_sdpa_with_explicit_mask(nq, nk, causal):
    rng = np.random.default_rng(nq * 1000 + nk + causal)
    d = 16
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    o, lse = oracle.forward_decode(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, _sdpa_masked(q, k, v, 0.3, causal), rtol=1e-12, atol=1e-12)
    s = 0.3 * torch.tensor(q) @ torch.tensor(k).T
    if causal:
        s[torch.arange(nk)[None, :] > torch.arange(nk - nq, nk)[:, None]] = -math.inf
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(3)
    n, d = 40, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = oracle.forward_decode(q, k, v, 0.5, True)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)
    o1c, l1c = oracle.forward_decode(q[:1], k, v, 0.5, True)
    o1n, l1n = oracle.forward_decode(q[:1], k, v, 0.5, False)
    np.testing.assert_array_equal(o1c, o1n)
    np.testing.assert_array_equal(l1c, l1n)
    with pytest.raises(ValueError):
        oracle.forward_decode(q, k[:10], v[:10], 0.5, True)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_heads_matches_sdpa_gqa(causal):
    rng = np.random.default_rng(11)
    H, Hkv, nq, nk, d = 8, 2, 3, 50, 16
    q, k, v = _rand(rng, H, nq, d), _rand(rng, Hkv, nk, d), _rand(rng, Hkv, nk, d)
    o, _ = oracle.forward_decode_heads(q, k, v, 0.25, causal)
    np.testing.assert_allclose(o, _sdpa_masked(q, k, v, 0.25, causal), rtol=1e-12, atol=1e-12)


def test_merge_reproduces_the_worked_example():
    g = json.load(open(GOLDEN))
    s1, s2 = np.array(g["first_block_scores"]), np.array(g["second_block_scores"])
    vals = np.array(g["values"])
    v1, v2 = vals[:3, None], vals[3:, None]
    # each block alone, by its own closed form
    lse1, lse2 = math.log(np.exp(s1).sum()), math.log(np.exp(s2).sum())
    o1 = (np.exp(s1 - lse1)[:, None] * v1).sum(0)
    o2 = (np.exp(s2 - lse2)[:, None] * v2).sum(0)
    o, lse = oracle.merge_partials(np.stack([o1, o2])[:, None, :], np.array([[lse1], [lse2]]))
    # one-shot closed forms over all four scores
    allv = np.concatenate([s1, s2])
    lse_ref = math.log(np.exp(allv).sum())
    o_ref = (np.exp(allv - lse_ref) * vals).sum()
    assert abs(lse[0] - lse_ref) <= 1e-15 * abs(lse_ref)
    assert abs(o[0, 0] - o_ref) <= 1e-14 * abs(o_ref)
    assert abs(lse[0] - 4.440189698561196) < 1e-14
    assert abs(o[0, 0] - 34.92652734585769) < 1e-13
    # the weight of the first block is its rescale e^(3 - 4) times its own
    # denominator over the new one
    w1 = math.exp(lse1 - lse[0])
    l1 = np.exp(s1 - 3).sum()
    assert abs(w1 - math.exp(g["rescale_exponent"]) * l1 / (math.exp(-1) * l1 + 1)) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[0, 50], [0, 17, 50], [0, 1, 2, 30, 31, 50], [0, 50, 50], [0, 0, 25, 50]])
def test_merge_of_disjoint_key_sets_is_the_whole(cuts, causal):
    rng = np.random.default_rng(len(cuts) + causal)
    nq, nk, d = 4, 50, 8
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    o_ref, lse_ref = oracle.forward_decode(q, k, v, 0.4, causal)
    # each part: the keys [a, b) with the same per-query visibility
    parts_o, parts_l = [], []
    pos = np.arange(nk - nq, nk)
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = 0.4 * q @ k[a:b].T
        if causal:
            s[np.arange(a, b)[None, :] > pos[:, None]] = -np.inf
        if b == a:
            s = np.full((nq, 0), -np.inf)
        p, l = oracle.softmax_rows(s) if b > a else (np.zeros((nq, 0)), np.full(nq, -np.inf))
        parts_o.append(p @ v[a:b])
        parts_l.append(l)
    o, lse = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
    # the order of the parts does not matter
    perm = rng.permutation(len(parts_o))
    o2, lse2 = oracle.merge_partials(np.stack(parts_o)[perm], np.stack(parts_l)[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)


def test_merge_of_nothing_visible():
    o, lse = oracle.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(5)
    nq, nk, d = 3, 20, 8
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    good, _ = oracle.forward_decode(q, k, v, 0.5, True)
    # a mask off by one (queries placed one position earlier)
    real_scores = decode_mod.scores
    monkeypatch.setattr(decode_mod, "scores", lambda qr, kk, sc, pos, c: real_scores(qr, kk, sc, pos - 1, c))
    bad, _ = decode_mod.forward_decode(q, k, v, 0.5, True)
    assert not np.allclose(bad, good, atol=1e-6)
    monkeypatch.undo()
    # merges with a dropped normalisation or a dropped weight do not pass the
    # whole-from-parts check that merge_partials passes
    s_all = 0.5 * q @ k.T
    s_all[np.arange(nk)[None, :] > np.arange(nk - nq, nk)[:, None]] = -np.inf
    parts = []
    for a, b in ((0, 7), (7, 20)):
        p, l = oracle.softmax_rows(s_all[:, a:b])
        parts.append((p @ v[a:b], l))
    o_parts = np.stack([x for x, _ in parts])
    lse_parts = np.stack([l for _, l in parts])
    m = lse_parts.max(0)
    unnormalised = np.einsum("sr,srd->rd", np.exp(lse_parts - m), o_parts)
    unweighted = o_parts.mean(0)
    merged, _ = oracle.merge_partials(o_parts, lse_parts)
    np.testing.assert_allclose(merged, good, rtol=1e-12, atol=1e-12)
    assert not np.allclose(unnormalised, good, atol=1e-6)
    assert not np.allclose(unweighted, good, atol=1e-6)
