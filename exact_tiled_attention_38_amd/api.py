"""Python binding of libfa.so: tensor checks, output allocation, stream handoff.

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels. There is no other code path:
if the library is missing or a check fails, these functions raise.
"""

import ctypes
import math

import torch

from . import _lib

__all__ = ["forward", "forward_f32", "forward_fp8", "forward_block_sparse", "backward", "backward_workspace_bytes", "decode",
           "decode_workspace_bytes", "decode_noalloc", "DECODE_SCRATCH_BYTES", "merge", "status_string", "SPARSE_BLOCK_M", "SPARSE_BLOCK_N"]

# Block sizes of the block-sparse selection (FA_SPARSE_BLOCK_M / _N in include/fa.h).
SPARSE_BLOCK_M = 256
SPARSE_BLOCK_N = 64


def status_string(code):
    return _lib.status_string(code)


def _stream(t):
    """The HIP stream PyTorch currently uses on t's device (work is enqueued there)."""
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(tensors, names, dtype, shape=None):
    ref = tensors[0]
    if shape is None:
        if ref.dim() != 4:
            raise ValueError(f"{names[0]} must be [B, H, N, d], got shape {tuple(ref.shape)}")
        shape = tuple(ref.shape)
    for t, n in zip(tensors, names):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{n} must be on a GPU device, got {t.device}")
        if t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, expected {ref.device}")
        if t.dtype != dtype:
            raise TypeError(f"{n} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shape}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    return shape


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _kv_heads(q, k, v):
    """Shape of q and the key/value head count: k and v are [B, Hkv, N, d], Hkv | H."""
    B, H, N, d = _check([q], ["q"], torch.bfloat16)
    if k.dim() != 4:
        raise ValueError(f"k must be [B, Hkv, N, d], got shape {tuple(k.shape)}")
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"k/v have {Hkv} heads, which must divide q's {H} heads")
    _check([k, v], ["k", "v"], torch.bfloat16, (B, Hkv, N, d))
    if k.device != q.device:
        raise ValueError(f"k is on {k.device}, expected {q.device}")
    return B, H, Hkv, N, d


def forward(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Exact attention forward on bf16 tensors. Returns (o, lse).

    q is [B, H, N, d]; k and v are [B, Hkv, N, d] with Hkv dividing H (Hkv = H
    is ordinary multi-head attention; fewer key/value heads are shared by
    consecutive query heads). o is bf16 [B, H, N, d]; lse is fp32 [B, H, N]
    (natural-log logsumexp of the scaled, masked score row). scale defaults
    to 1/sqrt(d). `out` and `lse` may be passed to write into preallocated
    tensors.
    """
    B, H, Hkv, N, d = _kv_heads(q, k, v)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check([o], ["out"], torch.bfloat16, (B, H, N, d))
    _check([l], ["lse"], torch.float32, (B, H, N))
    if o.device != q.device or l.device != q.device:
        raise ValueError(f"out and lse must be on {q.device}")
    if Hkv == H:
        rc = _lib.lib().fa_forward(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
            B, H, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
        )
        _lib.check(rc, "fa_forward")
    else:
        rc = _lib.lib().fa_forward_gqa(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
            B, H, Hkv, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
        )
        _lib.check(rc, "fa_forward_gqa")
    return o, l


def forward_f32(q, k, v, causal=False, scale=None):
    """Exact attention forward with fp32 inputs, arithmetic and output. Returns (o, lse)."""
    B, H, N, d = _check([q, k, v], ["q", "k", "v"], torch.float32)
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.lib().fa_forward_f32(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
        B, H, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_forward_f32")
    return o, l


def backward_workspace_bytes(B, H, N, d):
    return int(_lib.lib().fa_backward_workspace_bytes(B, H, N, d))


def backward(q, k, v, o, do, lse, causal=False, scale=None, workspace=None):
    """Gradients (dq, dk, dv) of exact attention, recomputing P from lse.

    q, o, do: bf16 [B, H, N, d]; k, v: bf16 [B, Hkv, N, d] (Hkv | H, as in
    forward()); lse: fp32 [B, H, N] from forward(). dk and dv have k's shape:
    a shared key/value head receives the sum over its query heads. A
    workspace of backward_workspace_bytes() bytes is allocated unless given.
    """
    B, H, Hkv, N, d = _kv_heads(q, k, v)
    _check([q, o, do], ["q", "o", "do"], torch.bfloat16)
    _check([lse], ["lse"], torch.float32, (B, H, N))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = backward_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes or workspace.device != q.device:
        raise ValueError(f"workspace must hold {nbytes} bytes on {q.device}")
    rc = _lib.lib().fa_backward_gqa(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        B, H, Hkv, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_backward_gqa")
    return dq, dk, dv


def decode_workspace_bytes(B, H, Hkv, Nq, Nk, d):
    return int(_lib.lib().fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d))


def decode(q, k, v, causal=False, scale=None, workspace=None, out=None, lse=None):
    """Attention of a few new queries against a cached sequence. Returns (o, lse).

    q: bf16 [B, H, Nq, d], the last Nq positions of the sequence; k, v: bf16
    [B, Hkv, Nk, d] with Hkv dividing H. causal: query i sees keys
    j <= Nk - Nq + i. A workspace of decode_workspace_bytes() bytes is
    allocated unless given.
    """
    B, H, Nq, d = _check([q], ["q"], torch.bfloat16)
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k must be [B, Hkv, Nk, d] with B={B}, d={d}; got {tuple(k.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"k/v have {Hkv} heads, which must divide q's {H} heads")
    _check([k, v], ["k", "v"], torch.bfloat16, (B, Hkv, Nk, d))
    if k.device != q.device:
        raise ValueError(f"k is on {k.device}, expected {q.device}")
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check([o], ["out"], torch.bfloat16, (B, H, Nq, d))
    _check([l], ["lse"], torch.float32, (B, H, Nq))
    nbytes = decode_workspace_bytes(B, H, Hkv, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes or workspace.device != q.device:
        raise ValueError(f"workspace must hold {nbytes} bytes on {q.device}")
    rc = _lib.lib().fa_decode(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), workspace.data_ptr(),
        B, H, Hkv, Nq, Nk, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_decode")
    return o, l


# Largest decode workspace the allocation-free decode can hold
# (FA_DECODE_SCRATCH_BYTES in include/fa.h).
DECODE_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q, k, v, out, lse, causal=False, scale=None):
    """decode() into preallocated `out` and `lse`, with no device allocation by
    the library or this binding: the key-split partials live in the library's
    static per-device scratch (DECODE_SCRATCH_BYTES; larger problems raise).
    Calls that may overlap on one GPU race on that scratch. Returns (out, lse)."""
    B, H, Nq, d = _check([q], ["q"], torch.bfloat16)
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k must be [B, Hkv, Nk, d] with B={B}, d={d}; got {tuple(k.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"k/v have {Hkv} heads, which must divide q's {H} heads")
    _check([k, v], ["k", "v"], torch.bfloat16, (B, Hkv, Nk, d))
    _check([out], ["out"], torch.bfloat16, (B, H, Nq, d))
    _check([lse], ["lse"], torch.float32, (B, H, Nq))
    for t, n in ((k, "k"), (out, "out"), (lse, "lse")):
        if t.device != q.device:
            raise ValueError(f"{n} is on {t.device}, expected {q.device}")
    rc = _lib.lib().fa_decode_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, H, Hkv, Nq, Nk, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_decode_noalloc")
    return out, lse


def merge(o_parts, lse_parts):
    """Merge partial results over disjoint key sets. Returns (o, lse).

    o_parts: bf16 [S, *rows_shape, d]; lse_parts: fp32 [S, *rows_shape] (natural
    log, as forward() returns it). o has shape [*rows_shape, d], lse [*rows_shape].
    """
    if o_parts.dim() < 3:
        raise ValueError("o_parts must be [S, ..., d]")
    S, d = o_parts.shape[0], o_parts.shape[-1]
    rows_shape = tuple(o_parts.shape[1:-1])
    _check([o_parts], ["o_parts"], torch.bfloat16, tuple(o_parts.shape))
    _check([lse_parts], ["lse_parts"], torch.float32, (S,) + rows_shape)
    if lse_parts.device != o_parts.device:
        raise ValueError(f"lse_parts is on {lse_parts.device}, expected {o_parts.device}")
    rows = 1
    for x in rows_shape:
        rows *= x
    o = torch.empty(rows_shape + (d,), dtype=torch.bfloat16, device=o_parts.device)
    l = torch.empty(rows_shape, dtype=torch.float32, device=o_parts.device)
    rc = _lib.lib().fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), o.data_ptr(), l.data_ptr(),
                             S, rows, d, _stream(o_parts))
    _lib.check(rc, "fa_merge")
    return o, l


def forward_block_sparse(q, k, v, row_ptr, cols, causal=False, scale=None):
    """Attention restricted to selected (query block, key block) pairs. Returns (o, lse).

    q: bf16 [B, H, N, d]; k, v: bf16 [B, Hkv, N, d]. The selection is in
    compressed-row form over the B * H * ceil(N / SPARSE_BLOCK_M) query blocks
    (b-major, then h, then block): row_ptr int32 [rows + 1] and cols int32 [nnz]
    key-block indices (blocks of SPARSE_BLOCK_N keys), both on q's device.
    Rows that see no key get o = 0 and lse = -inf.
    """
    B, H, Hkv, N, d = _kv_heads(q, k, v)
    n_rows = B * H * -(-N // SPARSE_BLOCK_M)
    for t, name in ((row_ptr, "row_ptr"), (cols, "cols")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 1-D int32 tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, expected {q.device}")
    if row_ptr.numel() != n_rows + 1:
        raise ValueError(f"row_ptr must have {n_rows + 1} entries, got {row_ptr.numel()}")
    nnz = cols.numel()
    cols_arg = cols if nnz > 0 else row_ptr  # any valid device pointer when the list is empty
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.lib().fa_forward_block_sparse(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), row_ptr.data_ptr(),
        cols_arg.data_ptr(), nnz, B, H, Hkv, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_forward_block_sparse")
    return o, l


def forward_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, scale=None):
    """Exact attention of fp8 (e4m3) inputs with per-tensor dequantisation factors. Returns (o, lse).

    q: torch.float8_e4m3fn [B, H, N, 128]; k, v: [B, Hkv, N, 128]. The values
    attended are code * descale. o is bf16 [B, H, N, 128], lse fp32 [B, H, N].
    """
    B, H, N, d = _check([q], ["q"], torch.float8_e4m3fn)
    if k.dim() != 4:
        raise ValueError(f"k must be [B, Hkv, N, d], got shape {tuple(k.shape)}")
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"k/v have {Hkv} heads, which must divide q's {H} heads")
    _check([k, v], ["k", "v"], torch.float8_e4m3fn, (B, Hkv, N, d))
    if k.device != q.device:
        raise ValueError(f"k is on {k.device}, expected {q.device}")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = _lib.lib().fa_forward_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
        float(q_descale), float(k_descale), float(v_descale),
        B, H, Hkv, N, d, int(bool(causal)), _scale(scale, d), _stream(q),
    )
    _lib.check(rc, "fa_forward_fp8")
    return o, l
