"""Exact tiled attention for AMD MI355X (gfx950).

Forward and backward of exact dense softmax attention, computed by hand-written
HIP kernels in libfa.so (C ABI declared in include/fa.h). This package is the
thin Python binding: it checks tensors, allocates outputs with PyTorch and
passes device pointers and the current stream to the library.
"""

from .api import (DECODE_SCRATCH_BYTES, SPARSE_BLOCK_M, SPARSE_BLOCK_N, backward, backward_workspace_bytes,
                  decode, decode_noalloc, decode_workspace_bytes, forward, forward_block_sparse, forward_f32,
                  forward_fp8, merge, status_string)

__all__ = ["forward", "forward_f32", "forward_fp8", "forward_block_sparse", "backward", "backward_workspace_bytes", "decode",
           "decode_workspace_bytes", "decode_noalloc", "merge", "status_string", "SPARSE_BLOCK_M", "SPARSE_BLOCK_N",
           "DECODE_SCRATCH_BYTES"]
