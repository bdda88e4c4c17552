"""Plain fp64 CPU oracle for exact dense softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
cpu_baseline leg of the benchmark may import this module. The library in
exact_tiled_attention_38_amd/ never imports it, and this module imports
nothing from that library: the two share no code.

What it computes, per (batch, head) slice with Q, K, V of shape [N, d]:

  Sources (three web pages; cited by title and section):
    [KVC] "Attention and KV Compression" (katajob.com), sections
          "Tiling and online softmax", "Recomputation in the backward pass",
          "What it does and does not change".
    [D19] "FlashAttention — how 100K-token attention fits in memory"
          (llmdaily.org, day 19): the softmax equation in
          "But softmax needs the whole row — right?".
    [TL]  "FlashAttention" (tensorlab.fun flagship module), Beat 01
          "What problem existed?": standard attention is four operations,
          score, mask, softmax, weight.

  The method is exact: the tiled, online-softmax kernel is meant to reach the
  one-shot dense result up to floating-point reassociation ([KVC] "Tiling and
  online softmax" and "What it does and does not change"; [D19] "Why exact
  matters"). So this oracle is that one-shot definition written out, in fp64,
  with the full score row of every query materialised:

    1. score    S = scale * Q K^T                      ([TL] Beat 01; the
                                                        pages' softmax has no
                                                        scale, so the caller
                                                        passes one, 1/sqrt(d)
                                                        by default)
    2. mask     causal: S[i, j] = -inf for key j > query i ([TL] names a mask
                step without defining it; causal is read as "key j is
                visible to query i iff j <= i", equal query and key
                counts; non-causal means no mask)
    3. softmax  P[i, :] = exp(S[i, :] - m_i) / l_i,  m_i = max_j S[i, j],
                l_i = sum_j exp(S[i, j] - m_i)       ([D19] softmax equation,
                                                        max-subtracted as in
                                                        [KVC] for stability)
    4. weight   O = P V                              ([TL] Beat 01)
    5. lse_i = m_i + ln l_i, natural log, in scaled-score units: the
       "small per-row statistic" of [KVC] "Tiling and online softmax",
       read as one logsumexp per query row.

  Backward (the pages give no formula; [KVC] "Recomputation in the backward
  pass" says only that it is computed from Q, K, V and the saved statistics).
  Differentiating steps 1-4 gives, with upstream gradient dO:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_k dO[i, k] O[i, k]        (equals sum_j P[i, j] dP[i, j])
    dS = P * (dP - D[:, None])
    dQ = scale * dS K
    dK = scale * dS^T Q

Rows are processed in chunks only to bound host memory (a full 16K x 16K
fp64 head would be 2 GiB); every row still uses its complete score row, and
rows are independent, so chunking changes nothing in the arithmetic.

Fully masked rows cannot occur when the number of queries equals the number
of keys and key j is visible to query i iff j <= i. If a row ever has no
visible key, this oracle returns O = 0 and lse = -inf for it.
"""

import numpy as np

__all__ = ["scores", "softmax_rows", "forward", "backward"]


def _f64(x):
    """Exact upcast to fp64 (bf16 and fp32 values are representable)."""
    return np.asarray(x, dtype=np.float64)


def scores(q_rows, k, scale, row_index, causal):
    """Steps 1 and 2 ([TL] Beat 01: score, mask) for a set of query rows.

    q_rows: [R, d] query vectors; k: [N, d] all keys of the head;
    row_index: [R] integer position of each query row in the sequence.
    Returns the [R, N] fp64 score rows with masked entries set to -inf.
    """
    s = scale * (_f64(q_rows) @ _f64(k).T)
    if causal:
        key_index = np.arange(k.shape[0])
        s[key_index[None, :] > np.asarray(row_index)[:, None]] = -np.inf
    return s


def softmax_rows(s):
    """Step 3 ([D19] softmax equation, max-subtracted) and step 5 (lse).

    s: [R, N] score rows, -inf where masked.
    Returns (P [R, N], lse [R]).
    """
    s = _f64(s)
    m = s.max(axis=1)
    visible = np.isfinite(m)
    m_safe = np.where(visible, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    l_safe = np.where(visible, l, 1.0)
    p = e / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(visible, m + np.log(l_safe), -np.inf)
    return p, lse


def forward(q, k, v, scale, causal, rows=None, chunk=256):
    """O and lse of exact softmax attention for the given query rows of one head.

    q, k, v: [N, d] arrays (any float dtype; upcast exactly to fp64).
    rows: None for all rows, else an integer array of query positions.
    Returns (O [R, d] fp64, lse [R] fp64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    for c0 in range(0, rows.shape[0], chunk):
        r = rows[c0:c0 + chunk]
        p, lse[c0:c0 + chunk] = softmax_rows(scores(q[r], k, scale, r, causal))
        o[c0:c0 + chunk] = p @ v  # step 4, weight
    return o, lse


def backward(q, k, v, do, scale, causal, chunk=256):
    """Analytic fp64 gradients of exact softmax attention for one head.

    q, k, v, do: [N, d]. Returns (dq, dk, dv, o, lse), all fp64, where o and
    lse are this oracle's own forward results (D uses the oracle's O).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for c0 in range(0, n, chunk):
        r = np.arange(c0, min(n, c0 + chunk))
        p, lse[r] = softmax_rows(scores(q[r], k, scale, r, causal))
        o[r] = p @ v
        dv += p.T @ do[r]
        dp = do[r] @ v.T
        d_row = np.sum(do[r] * o[r], axis=1)
        ds = p * (dp - d_row[:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv, o, lse
