"""Pins for the fp64 CPU oracle (oracle/), checked against things other than itself.

Each pin comes from the pages or from mathematics:
  * the worked online-softmax example printed in "FlashAttention — how
    100K-token attention fits in memory" (llmdaily.org, day 19), section
    "Online softmax intuition" (tests/golden/online_softmax_worked_example.json);
  * the softmax definition in the same page's section "But softmax needs the
    whole row — right?": probability rows sum to one; all-ones values give
    all-ones outputs; a per-row shift of the scores changes nothing but lse;
  * the exactness claim of "Attention and KV Compression" (katajob.com),
    section "Tiling and online softmax": the blockwise online softmax equals
    the one-shot result (here in fp64, at several block sizes, ragged);
  * a library routine the definition reduces to: PyTorch's fp64 CPU
    scaled_dot_product_attention and logsumexp;
  * brute force with Python loops and math.exp on tiny inputs;
  * closed forms: one key gives O = V_0 and lse = scale * q.k;
  * calculus for the backward: central finite differences, PyTorch autograd
    and the invariants sum_j dS_ij = 0, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
Finally, mistakes planted in the oracle (on the CPU) must trip these pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_worked_example.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- worked example


def test_worked_example_online_softmax():
    g = json.load(open(GOLDEN))
    s1, s2, v = g["first_block_scores"], g["second_block_scores"], g["values"]
    o, lse, trace = oracle.online_softmax_row([s1, s2], [v[:3], v[3:]])
    # first block: max 3, denominator relative to that max
    assert trace[0]["m"] == g["first_block_max"]
    l1 = math.exp(1 - 3) + math.exp(2 - 3) + math.exp(3 - 3)
    assert trace[0]["l"] == pytest.approx(l1, rel=1e-15)
    # a later block holding 4 raises the max to 4 and rescales by e^(3-4) = e^-1
    assert trace[1]["m"] == g["new_max"]
    assert trace[1]["alpha"] == math.exp(g["rescale_exponent"])
    acc1 = sum(math.exp(s - 3) * x for s, x in zip(s1, v[:3]))
    assert float(trace[0]["acc"]) == pytest.approx(acc1, rel=1e-15)
    assert trace[1]["l"] == pytest.approx(math.exp(-1) * l1 + 1.0, rel=1e-15)
    assert float(trace[1]["acc"]) == pytest.approx(math.exp(-1) * acc1 + v[3], rel=1e-15)
    # closed forms over the whole row [1, 2, 3, 4]
    row = s1 + s2
    z = sum(math.exp(s) for s in row)
    p = [math.exp(s) / z for s in row]
    assert lse == pytest.approx(math.log(z), rel=1e-15)
    assert float(o) == pytest.approx(sum(pi * x for pi, x in zip(p, v)), rel=1e-15)
    # the one-shot oracle on the same row agrees
    p_one, lse_one = oracle.softmax_rows(np.array([row]))
    np.testing.assert_allclose(p_one[0], p, rtol=1e-15)
    assert lse_one[0] == pytest.approx(math.log(z), rel=1e-15)


# ---------------------------------------------------------------- softmax definition


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    rng = np.random.default_rng(1)
    n, d = 97, 16
    q, k = _rand(rng, n, d) * 3, _rand(rng, n, d)
    s = oracle.scores(q, k, 0.25, np.arange(n), causal)
    p, _ = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(p >= 0)


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_values_give_all_ones_output(causal):
    rng = np.random.default_rng(2)
    n, d = 65, 8
    q, k = _rand(rng, n, d) * 4, _rand(rng, n, d)
    o, _ = oracle.forward(q, k, np.ones((n, d)), 1 / math.sqrt(d), causal)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)


def test_causal_visibility_pattern():
    rng = np.random.default_rng(3)
    n, d = 40, 4
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    p, _ = oracle.softmax_rows(oracle.scores(q, k, 0.5, np.arange(n), True))
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.all(p[j > i] == 0.0)
    assert np.all(p[j <= i] > 0.0)


def test_shift_invariance():
    rng = np.random.default_rng(4)
    s = _rand(rng, 7, 50) * 5
    c = _rand(rng, 7) * 100
    p0, lse0 = oracle.softmax_rows(s)
    p1, lse1 = oracle.softmax_rows(s + c[:, None])
    np.testing.assert_allclose(p1, p0, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse1, lse0 + c, rtol=1e-13)


def test_large_scores_are_stable():
    # scores far beyond exp's fp64 range: the max subtraction keeps it finite
    s = np.array([[1000.0, 999.0, -1000.0], [-800.0, -801.0, -802.0]])
    p, lse = oracle.softmax_rows(s)
    assert np.all(np.isfinite(p)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(lse[0], 1000.0 + math.log(1 + math.exp(-1) + math.exp(-2000)), rtol=1e-15)


def test_fully_masked_row_gives_zero_output_and_minus_inf_lse():
    s = np.array([[-np.inf, -np.inf], [0.0, -np.inf]])
    p, lse = oracle.softmax_rows(s)
    assert np.all(p[0] == 0) and lse[0] == -np.inf
    assert p[1, 0] == 1.0 and lse[1] == 0.0


# ---------------------------------------------------------------- blockwise == one-shot


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 3, 7, 64, 10**9])
def test_blockwise_equals_oneshot(causal, block):
    rng = np.random.default_rng(5 + block % 97)
    n, d = 131, 12  # 131 = ragged for every block size above except 1
    q = _rand(rng, n, d) * 4  # large, shifting row maxima exercise the rescale
    k, v = _rand(rng, n, d), _rand(rng, n, d)
    scale = 1 / math.sqrt(d)
    o1, lse1 = oracle.forward(q, k, v, scale, causal)
    o2, lse2 = oracle.blockwise_forward(q, k, v, scale, causal, min(block, n))
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse1, rtol=1e-12, atol=1e-13)


def test_row_subset_matches_full_rows():
    rng = np.random.default_rng(6)
    n, d = 300, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    rows = np.array([0, 1, 17, 255, 256, 299])
    o_all, lse_all = oracle.forward(q, k, v, 0.3, True, chunk=64)
    o_sub, lse_sub = oracle.forward(q, k, v, 0.3, True, rows=rows, chunk=4)
    np.testing.assert_array_equal(o_sub, o_all[rows])
    np.testing.assert_array_equal(lse_sub, lse_all[rows])


# ---------------------------------------------------------------- library routine / brute force


def _sdpa_reference(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        n = q.shape[0]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return o[0, 0].numpy(), torch.logsumexp(s, dim=-1)[0, 0].numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 17, 63, 64, 65, 127, 129, 257])
@pytest.mark.parametrize("d", [1, 4, 64, 128])
def test_matches_torch_sdpa_fp64(n, d, causal):
    rng = np.random.default_rng(1000 * n + d)
    q, k, v = _rand(rng, n, d) * 2, _rand(rng, n, d), _rand(rng, n, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, scale, causal, chunk=50)
    o_ref, lse_ref = _sdpa_reference(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def _python_bruteforce(q, k, v, scale, causal):
    n, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        z = sum(math.exp(x) for x in s)
        out.append([sum(math.exp(x) / z * v[j][c] for x, j in zip(s, keys)) for c in range(d)])
        lses.append(math.log(z))
    return out, lses


@pytest.mark.parametrize("causal", [False, True])
def test_matches_python_loop_bruteforce(causal):
    rng = np.random.default_rng(7)
    n, d = 6, 3
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o_ref, lse_ref = _python_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    o, lse = oracle.forward(q, k, v, 0.7, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)


def test_single_key_closed_form():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 64), _rand(rng, 1, 64), _rand(rng, 1, 64)
    for causal in (False, True):
        o, lse = oracle.forward(q, k, v, 0.125, causal)
        np.testing.assert_array_equal(o, v)
        assert lse[0] == pytest.approx(0.125 * float(q[0] @ k[0]), rel=1e-15)


def test_identical_keys_give_mean_of_values():
    # every score in a row equal: P is uniform, O is the mean of visible values
    rng = np.random.default_rng(9)
    n, d = 20, 5
    q, v = _rand(rng, n, d), _rand(rng, n, d)
    k = np.tile(_rand(rng, 1, d), (n, 1))
    o, lse = oracle.forward(q, k, v, 0.5, True)
    csum = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, csum, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]) + np.log(np.arange(1, n + 1)), rtol=1e-13)


# ---------------------------------------------------------------- backward


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.forward(q, k, v, scale, causal)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_finite_differences(causal):
    rng = np.random.default_rng(10)
    n, d = 9, 5
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 0.6
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, scale, causal, chunk=4)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            fm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_directional_finite_differences(causal):
    rng = np.random.default_rng(11)
    n, d = 33, 16
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 1 / math.sqrt(d)
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, scale, causal, chunk=8)
    for _ in range(3):
        eq, ek, ev = (_rand(rng, n, d) for _ in range(3))
        h = 1e-6
        fp = _loss(q + h * eq, k + h * ek, v + h * ev, do, scale, causal)
        fm = _loss(q - h * eq, k - h * ek, v - h * ev, do, scale, causal)
        num = (fp - fm) / (2 * h)
        ana = np.sum(dq * eq) + np.sum(dk * ek) + np.sum(dv * ev)
        assert ana == pytest.approx(num, rel=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    rng = np.random.default_rng(12)
    n, d = 70, 32
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x[None, None], requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.from_numpy(do)[None, None])
    dq, dk, dv, o, _ = oracle.backward(q, k, v, do, scale, causal, chunk=16)
    np.testing.assert_allclose(o, to.detach()[0, 0].numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    rng = np.random.default_rng(13)
    n, d = 50, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 0.4
    dq, dk, dv, o, _ = oracle.backward(q, k, v, do, scale, causal, chunk=16)
    # sum_j dK_j = scale * sum_i q_i * (sum_j dS_ij) = 0, since every dS row sums to 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # sum_j dV_j = sum_i (sum_j P_ij) dO_i = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    # row sums of dS vanish
    p, _ = oracle.softmax_rows(oracle.scores(q, k, scale, np.arange(n), causal))
    ds = p * ((do @ v.T) - np.sum(do * o, axis=1)[:, None])
    np.testing.assert_allclose(ds.sum(axis=1), 0.0, atol=1e-13)
    # dQ depends on K only through dS rows: a shift of every key by a constant vector
    # shifts each score row by a constant and leaves O and dV unchanged
    c = _rand(rng, d)
    dq2, dk2, dv2, o2, _ = oracle.backward(q, k + c, v, do, scale, causal, chunk=16)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk2, dk, rtol=1e-10, atol=1e-12)


def test_backward_single_key_closed_form():
    # one key: P = 1, O = V_0, so dV_0 = dO_0 and every other gradient is zero
    rng = np.random.default_rng(14)
    q, k, v, do = (_rand(rng, 1, 6) for _ in range(4))
    dq, dk, dv, o, lse = oracle.backward(q, k, v, do, 0.3, True)
    np.testing.assert_array_equal(dv, do)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


# ---------------------------------------------------------------- planted mistakes


def _pins_pass():
    """Run a compact set of the pins above on the (possibly patched) oracle."""
    try:
        for causal in (False, True):
            rng = np.random.default_rng(15)
            n, d = 33, 8
            q, k, v, do = (_rand(rng, n, d) for _ in range(4))
            scale = 1 / math.sqrt(d)
            o, lse = oracle_attention.forward(q, k, v, scale, causal)
            o_ref, lse_ref = _sdpa_reference(q, k, v, scale, causal)
            np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(lse, lse_ref, rtol=1e-10, atol=1e-11)
            dq, dk, dv, _, _ = oracle_attention.backward(q, k, v, do, scale, causal)
            eq, ek, ev = (_rand(rng, n, d) for _ in range(3))
            h = 1e-6
            f = lambda t: float(np.sum(do * oracle_attention.forward(q + t * eq, k + t * ek, v + t * ev, scale, causal)[0]))
            num = (f(h) - f(-h)) / (2 * h)
            ana = np.sum(dq * eq) + np.sum(dk * ek) + np.sum(dv * ev)
            assert abs(ana - num) <= 1e-6 * abs(num) + 1e-9
        return True
    except AssertionError:
        return False


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def _mutant_scores(kind):
    real = oracle_attention.scores

    def f(q_rows, k, scale, row_index, causal):
        if kind == "no_scale":
            return real(q_rows, k, 1.0, row_index, causal)
        if kind == "mask_off_by_one":
            s = real(q_rows, k, scale, row_index, False)
            if causal:
                key_index = np.arange(k.shape[0])
                s[key_index[None, :] >= np.asarray(row_index)[:, None]] = -np.inf
                s[:, 0] = np.where(np.isinf(s[:, 0]), 0.0, s[:, 0])
            return s
        if kind == "transposed":
            # S^T in place of S: query i scored against key j as k_i . q_j
            # (only meaningful when every row is requested at once, as the pins do)
            assert len(q_rows) == k.shape[0]
            qs, ks = np.asarray(q_rows, dtype=np.float64), np.asarray(k, dtype=np.float64)
            s = scale * (ks @ qs.T)
            if causal:
                key_index = np.arange(k.shape[0])
                s[key_index[None, :] > np.asarray(row_index)[:, None]] = -np.inf
            return s
        raise AssertionError(kind)

    return f


def _mutant_softmax(kind):
    real = oracle_attention.softmax_rows

    def f(s):
        p, lse = real(s)
        if kind == "lse_without_max":
            m = np.asarray(s).max(axis=1)
            return p, lse - m
        if kind == "unnormalised":
            e = np.exp(np.asarray(s) - np.asarray(s).max(axis=1)[:, None])
            return e, lse
        raise AssertionError(kind)

    return f


@pytest.mark.parametrize("kind", ["no_scale", "mask_off_by_one", "transposed"])
def test_planted_score_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle_attention, "scores", _mutant_scores(kind))
    assert not _pins_pass()


@pytest.mark.parametrize("kind", ["lse_without_max", "unnormalised"])
def test_planted_softmax_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle_attention, "softmax_rows", _mutant_softmax(kind))
    assert not _pins_pass()


@pytest.mark.parametrize("kind", ["ds_sign", "dk_without_scale", "dv_untransposed"])
def test_planted_backward_mistakes_are_caught(monkeypatch, kind):
    real = oracle_attention.backward

    def mutant(q, k, v, do, scale, causal, chunk=256):
        dq, dk, dv, o, lse = real(q, k, v, do, scale, causal, chunk)
        if kind == "ds_sign":
            return -dq, -dk, dv, o, lse
        if kind == "dk_without_scale":
            return dq, dk / scale, dv, o, lse
        if kind == "dv_untransposed":
            s = oracle_attention.scores(q, k, scale, np.arange(len(q)), causal)
            p, _ = oracle_attention.softmax_rows(s)
            return dq, dk, p @ np.asarray(do, dtype=np.float64), o, lse
        raise AssertionError(kind)

    monkeypatch.setattr(oracle_attention, "backward", mutant)
    assert not _pins_pass()
