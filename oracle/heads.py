"""fp64 CPU oracle for attention with shared key/value heads (grouped-query).

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU
library, and sharing no code with it.

"Attention and KV Compression" (katajob.com), section "The composability
point": sharing key/value heads between query heads only changes how many
K/V heads there are, and the tiled method runs over them unchanged. Read
plainly: query head h of H uses key/value
head h // (H / Hkv) of Hkv (consecutive query heads form a group), and each
query head's attention is exactly the single-head definition of
oracle/attention.py on its group's K and V. The gradient of a shared K or V
is the sum of the gradients it receives from the query heads of its group
(the chain rule over the shared input).
"""

import numpy as np

from .attention import backward as _backward_head
from .attention import forward as _forward_head

__all__ = ["kv_head", "forward_heads", "backward_heads"]


def kv_head(h, H, Hkv):
    """Key/value head read by query head h (H query heads, Hkv | H)."""
    if Hkv < 1 or H % Hkv:
        raise ValueError("the number of key/value heads must divide the number of query heads")
    return h // (H // Hkv)


def forward_heads(q, k, v, scale, causal, rows=None):
    """q: [H, N, d]; k, v: [Hkv, N, d]. Returns (O [H, R, d], lse [H, R])."""
    H, Hkv = q.shape[0], k.shape[0]
    outs = [_forward_head(q[h], k[kv_head(h, H, Hkv)], v[kv_head(h, H, Hkv)], scale, causal, rows=rows)
            for h in range(H)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def backward_heads(q, k, v, do, scale, causal):
    """Gradients for q: [H, N, d], k, v: [Hkv, N, d], do: [H, N, d].

    Returns (dq [H, N, d], dk [Hkv, N, d], dv [Hkv, N, d]), fp64.
    """
    H, Hkv = q.shape[0], k.shape[0]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for h in range(H):
        g = kv_head(h, H, Hkv)
        dq[h], dk_h, dv_h, _, _ = _backward_head(q[h], k[g], v[g], do[h], scale, causal)
        dk[g] += dk_h
        dv[g] += dv_h
    return dq, dk, dv
