"""fp64 CPU oracle pieces for the fp8 (e4m3) forward.

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU
library, and sharing no code with it.

"Attention and KV Compression" (katajob.com), section "What it does and does
not change": the method's later revisions also handle lower-precision
numbers. Reading: Q, K and V arrive as 8-bit floating point codes (the OCP
e4m3 format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, S.1111.111 is NaN, largest finite 448) together with one fp32
dequantisation factor per tensor; the attention being computed is the exact
one of the dequantised values, code * factor. So the oracle decodes the
codes by the format's definition, multiplies by the factors, and runs the
one-shot oracle of attention.py on the result in fp64.
"""

import numpy as np

from .attention import forward as _forward

__all__ = ["e4m3_decode", "forward_fp8"]


def e4m3_decode(codes):
    """uint8 e4m3 codes -> fp64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    subnormal = sign * (man / 8.0) * np.exp2(-6.0)
    out = np.where(exp == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def forward_fp8(q_codes, k_codes, v_codes, q_descale, k_descale, v_descale, scale, causal, rows=None):
    """Exact attention of the dequantised inputs of one head ([N, d] code arrays).

    Returns (O [R, d], lse [R]) in fp64; lse is that of the dequantised scores.
    """
    q = e4m3_decode(q_codes) * float(q_descale)
    k = e4m3_decode(k_codes) * float(k_descale)
    v = e4m3_decode(v_codes) * float(v_descale)
    return _forward(q, k, v, scale, causal, rows=rows)
