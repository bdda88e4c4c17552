"""Closed-form expectations of the bookkeeping probes (integer arithmetic only).

The probe inputs are workloads.probe_inputs / probe_heads_inputs. For every
query row these give the number of keys the row sees and the key index its
output spells, from the visibility rule alone:
  dense / decode: row i of Nq queries at the end of Nk keys sees keys
      [0, Nk - Nq + i] (causal) or [0, Nk);
  block-sparse: row i sees the keys of its query block's listed 64-key blocks
      that lie below N and, causal, at or below i.
tests/test_probe_expectations.py checks these against the fp64 oracle run on
the same probe inputs; the GPU tests compare the HIP path with them bit for
bit at full size.
"""

import numpy as np

from exact_tiled_attention_38_amd import workloads as W

SPARSE_BM, SPARSE_BN = 256, 64


def extreme_index(order, last, kind):
    """Index j in [0, last] maximising (kind "max") or minimising ("min") order[j],
    for each entry of the int array `last`; `order` is a permutation."""
    inv = np.empty_like(order)
    inv[order] = np.arange(order.shape[0])
    acc = np.maximum.accumulate(order) if kind == "max" else np.minimum.accumulate(order)
    return inv[acc[last]]


def dense_expected(kind, H, Hkv, Nq, Nk, causal, rotate=True):
    """(count, index), int64 [H, Nq]: visible keys per row and the spelled key."""
    i = np.arange(Nq, dtype=np.int64)
    last = (Nk - Nq + i) if causal else np.full(Nq, Nk - 1, dtype=np.int64)
    group = H // Hkv
    count = np.tile(last + 1, (H, 1))
    index = np.stack([extreme_index(W.probe_key_order(h // group if rotate else 0, Nk), last, kind)
                      for h in range(H)])
    return count, index


def sparse_expected(kind, N, row_ptr, cols, causal, n_heads, bm=SPARSE_BM, bn=SPARSE_BN):
    """(count, index), int64 [n_heads, N] for the un-rotated probes: visible keys per
    row and the largest (max) / smallest (min) visible key, -1 where a row sees none.
    row_ptr / cols: the CSR list over (head, query block), key blocks of bn keys."""
    n_qb = -(-N // bm)
    rows_total = n_qb * bm
    count = np.zeros((n_heads, rows_total), dtype=np.int64)
    hi = np.full((n_heads, rows_total), -1, dtype=np.int64)
    lo = np.full((n_heads, rows_total), np.iinfo(np.int64).max, dtype=np.int64)
    off = np.arange(bm, dtype=np.int64)
    n_kb = -(-N // bn)
    for hd in range(n_heads):
        r0 = hd * n_qb
        beg, end = int(row_ptr[r0]), int(row_ptr[r0 + n_qb])
        c = np.clip(cols[beg:end].astype(np.int64), 0, n_kb - 1)
        qb = np.repeat(np.arange(n_qb), np.diff(row_ptr[r0:r0 + n_qb + 1]).astype(np.int64))
        i = qb[:, None] * bm + off[None, :]
        k0 = np.broadcast_to((c * bn)[:, None], i.shape)
        k1 = np.minimum(k0 + bn, N)
        top = np.minimum(k1, i + 1) if causal else k1
        n = np.clip(top - k0, 0, None)
        rows = i.ravel()
        np.add.at(count[hd], rows, n.ravel())
        vis = (n > 0).ravel()
        np.maximum.at(hi[hd], rows[vis], (top - 1).ravel()[vis])
        np.minimum.at(lo[hd], rows[vis], k0.ravel()[vis])
    count, hi, lo = count[:, :N], hi[:, :N], lo[:, :N]
    lo = np.where(count == 0, -1, lo)
    return count, (hi if kind == "max" else lo)


def random_lists(rng, rows, n_kb, density, empty_every):
    """Seeded CSR selection: each row lists a random subset of key blocks in random
    order; every `empty_every`-th row is empty."""
    lists = []
    for r in range(rows):
        if empty_every and r % empty_every == empty_every - 1:
            lists.append([])
            continue
        lists.append(rng.permutation(rng.choice(n_kb, size=rng.binomial(n_kb, density), replace=False)).tolist())
    row_ptr = np.cumsum([0] + [len(x) for x in lists]).astype(np.int32)
    return row_ptr, np.array([c for x in lists for c in x], dtype=np.int32)
