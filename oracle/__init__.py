"""fp64 CPU oracle for exact dense softmax attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's cpu_baseline leg, never by the GPU library, and sharing no code
with it. See attention.py (the one-shot definition) and online_softmax.py
(the blockwise route used to pin it).
"""

from .attention import backward, forward, scores, softmax_rows
from .decode import forward_decode, forward_decode_heads, merge_partials
from .fp8 import e4m3_decode, forward_fp8
from .heads import backward_heads, forward_heads, kv_head
from .online_softmax import blockwise_forward, online_softmax_row
from .sparse import block_mask, forward_block_sparse

__all__ = [
    "forward",
    "backward",
    "scores",
    "softmax_rows",
    "blockwise_forward",
    "online_softmax_row",
    "kv_head",
    "forward_heads",
    "backward_heads",
    "forward_decode",
    "forward_decode_heads",
    "merge_partials",
    "block_mask",
    "forward_block_sparse",
    "e4m3_decode",
    "forward_fp8",
]
