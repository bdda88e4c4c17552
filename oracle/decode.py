"""fp64 CPU oracle for decode-shaped attention and for merging partial results.

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU
library, and sharing no code with it.

Decode. A few new queries (Nq, often 1) attend to a long cached sequence of
Nk keys. Reading: the queries are the last Nq positions of that sequence,
Nk - Nq .. Nk - 1, so with the causal mask query i sees keys
j <= Nk - Nq + i (with Nq = 1 it sees every key; with Nq = Nk this is the
ordinary causal mask). The result is the one-shot definition of
oracle/attention.py (score, mask, softmax, weight) at those positions.
"FlashAttention — how 100K-token attention fits in memory" (llmdaily.org,
day 19), section "Arithmetic intensity", contrasts prefill with decode: the
same computation with far less reuse per byte.

Merge. If the keys are split into disjoint sets and attention is computed
over each set alone, giving (O_s, lse_s) per row, the result over all keys
follows from the rescale identity of online softmax (same page, "Online
softmax intuition"; "Attention and KV Compression", "Tiling and online
softmax"): with M = max_s lse_s,
    lse = M + ln sum_s exp(lse_s - M),    O = sum_s exp(lse_s - lse) O_s.
A set with no visible key has lse_s = -inf and weight 0; a row with no
visible key in any set gets O = 0 and lse = -inf.
"""

import numpy as np

from .attention import scores, softmax_rows
from .heads import kv_head

__all__ = ["forward_decode", "forward_decode_heads", "merge_partials"]


def forward_decode(q, k, v, scale, causal):
    """q: [Nq, d] queries at positions Nk - Nq .. Nk - 1; k, v: [Nk, d].

    Returns (O [Nq, d], lse [Nq]) in fp64.
    """
    nq, nk = q.shape[0], k.shape[0]
    if causal and nq > nk:
        raise ValueError("causal decode needs Nq <= Nk")
    positions = np.arange(nk - nq, nk)
    p, lse = softmax_rows(scores(q, k, scale, positions, causal))
    return p @ np.asarray(v, dtype=np.float64), lse


def forward_decode_heads(q, k, v, scale, causal):
    """q: [H, Nq, d]; k, v: [Hkv, Nk, d] (query head h reads key/value head
    h // (H / Hkv)). Returns (O [H, Nq, d], lse [H, Nq])."""
    H, Hkv = q.shape[0], k.shape[0]
    outs = [forward_decode(q[h], k[kv_head(h, H, Hkv)], v[kv_head(h, H, Hkv)], scale, causal)
            for h in range(H)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def merge_partials(o_parts, lse_parts):
    """o_parts: [S, R, d] partial outputs, lse_parts: [S, R] their natural-log
    logsumexps (-inf where a part saw no key). Returns (O [R, d], lse [R])."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    seen = np.isfinite(m)
    m_safe = np.where(seen, m, 0.0)
    w = np.exp(lse_parts - m_safe[None, :])           # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    total_safe = np.where(seen, total, 1.0)
    with np.errstate(divide="ignore"):
        lse = np.where(seen, m + np.log(total_safe), -np.inf)
    o = np.einsum("sr,srd->rd", w / total_safe[None, :], o_parts)
    return o, lse
