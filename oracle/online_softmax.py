"""fp64 CPU blockwise (online-softmax) attention, used only to pin the oracle.

TEST INFRASTRUCTURE ONLY, like oracle/attention.py: only the test suite, the
smoke check and the benchmark's cpu_baseline leg may import it, and it shares
no code with the GPU library.

This is a second, independent route to the same numbers as the one-shot
oracle: it takes the online-softmax steps in the order the pages give them.

  [KVC] "Attention and KV Compression" (katajob.com), section "Tiling and
        online softmax": stream blocks of keys and values past a block of
        queries; carry a running maximum, a running sum of exponentials and
        a partial weighted sum of values; when a block raises the maximum,
        rescale the carried sum and output by the exponential of the
        difference, then add the block's contribution; at the end the
        accumulator equals the one-shot result.
  [D19] "FlashAttention — how 100K-token attention fits in memory"
        (llmdaily.org, day 19), sections "But softmax needs the whole row —
        right?" (running maximum, normalisation sum, weighted-V accumulator)
        and "Online softmax intuition" (worked example: first block [1, 2, 3]
        with maximum 3; a later block holding 4 rescales the carried
        accumulator by e^(3-4) = e^-1).

Agreement between this and the one-shot oracle is the pages' exactness claim
checked on the CPU in fp64.
"""

import math

import numpy as np

__all__ = ["online_softmax_row", "blockwise_forward"]


def online_softmax_row(score_blocks, value_blocks):
    """Online softmax over one query row, block by block.

    score_blocks: sequence of 1-D score arrays, one per key block, in order
                  (-inf marks a masked key).
    value_blocks: sequence of [len(block), dv] value arrays (or 1-D for a
                  scalar value per key).
    Returns (o, lse, trace). trace holds one dict per block with the running
    max m, the rescale factor alpha applied to what was carried in, the
    running denominator l and the running accumulator acc after the block.
    """
    m = -math.inf
    l = 0.0
    acc = None
    trace = []
    for s, v in zip(score_blocks, value_blocks):
        s = np.asarray(s, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        m_new = max(m, float(s.max()) if s.size else -math.inf)
        if m_new == -math.inf:  # nothing visible yet: carry on unchanged
            trace.append(dict(m=m, alpha=1.0, l=l, acc=acc))
            continue
        alpha = math.exp(m - m_new)  # e^(m_old - m_new); 0 on the first block
        p = np.exp(s - m_new)
        l = alpha * l + float(p.sum())
        contrib = np.tensordot(p, v, axes=(0, 0))
        acc = contrib if acc is None else alpha * acc + contrib
        m = m_new
        trace.append(dict(m=m, alpha=alpha, l=l, acc=acc))
    if acc is None:
        return None, -math.inf, trace
    return acc / l, m + math.log(l), trace


def blockwise_forward(q, k, v, scale, causal, block):
    """Blockwise attention for all rows of one head, keys streamed in blocks.

    q, k, v: [N, d]; block: key-block size (the last block may be ragged).
    All query rows are processed together; each key block is scored, masked,
    folded into the running (m, l, acc) of every row, then discarded.
    Returns (O [N, d], lse [N]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    for j0 in range(0, k.shape[0], block):
        j1 = min(k.shape[0], j0 + block)
        s = scale * (q @ k[j0:j1].T)  # this block's scores only
        if causal:
            keys = np.arange(j0, j1)
            s[keys[None, :] > rows[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        m_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - m_safe)  # 0 while nothing was visible
        p = np.exp(s - m_safe[:, None])  # masked keys give 0
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    visible = l > 0
    l_safe = np.where(visible, l, 1.0)
    o = acc / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(visible, m + np.log(l_safe), -np.inf)
    return o, lse
