"""fp64 CPU oracle for block-sparse attention (attention over selected blocks).

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU
library, and sharing no code with it.

"Attention and KV Compression" (katajob.com), section "The composability
point": with sparse selection the exact tiled kernel simply runs on the
blocks that were selected. Read plainly: the (query, key) plane of a head is
cut into blocks of block_m query rows by block_n keys; a selection lists, for
each query block, the key blocks it attends to; every (query, key) pair
outside the listed blocks is masked out (score -inf), and so is every pair
the causal mask removes when causal is set. The result is the one-shot
definition of oracle/attention.py (score, mask, softmax, weight) with that
mask. A row that sees no key at all gets O = 0 and lse = -inf.

The selection is in compressed-row form: the key blocks of query block r are
cols[row_ptr[r] : row_ptr[r + 1]].
"""

import numpy as np

from .attention import softmax_rows

__all__ = ["block_mask", "forward_block_sparse"]


def block_mask(n, row_ptr, cols, block_m, block_n, causal):
    """Boolean [n, n] visibility of one head: True where the pair is kept."""
    keep = np.zeros((n, n), dtype=bool)
    for r in range(len(row_ptr) - 1):
        for c in cols[row_ptr[r]:row_ptr[r + 1]]:
            keep[r * block_m:(r + 1) * block_m, c * block_n:(c + 1) * block_n] = True
    if causal:
        keep &= np.tril(np.ones((n, n), dtype=bool))
    return keep


def forward_block_sparse(q, k, v, scale, causal, row_ptr, cols, block_m, block_n, rows=None):
    """O and lse of one head ([N, d] inputs) restricted to the selected blocks.

    rows: None for every query row, else the query rows to return.
    Returns (O [R, d], lse [R]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
        keep = block_mask(n, row_ptr, cols, block_m, block_n, causal)
    else:
        # the same visibility, built for the requested rows only
        rows = np.asarray(rows, dtype=np.int64)
        keep = np.zeros((rows.shape[0], n), dtype=bool)
        key = np.arange(n)
        for a, i in enumerate(rows):
            r = i // block_m
            listed = np.zeros(n, dtype=bool)
            for c in cols[row_ptr[r]:row_ptr[r + 1]]:
                listed[c * block_n:(c + 1) * block_n] = True
            keep[a] = listed & ((key <= i) if causal else True)
    s = scale * (q[rows] @ k.T)
    s[~keep] = -np.inf
    p, lse = softmax_rows(s)
    return p @ v, lse
