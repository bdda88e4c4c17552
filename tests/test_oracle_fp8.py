"""Pins of the fp8 oracle (oracle/fp8.py), CPU only.

The e4m3 decoder is pinned by the format's landmark codes (largest finite
448, smallest normal 2^-6, smallest subnormal 2^-9, one, the NaN codes, the
sign bit) and, for all 256 codes, against PyTorch's own float8_e4m3fn
conversion; forward_fp8 is pinned against the dense oracle on values decoded
by PyTorch. A planted bias error (8 instead of 7) must be caught.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as fp8_mod


def test_landmark_codes():
    d = oracle.e4m3_decode
    assert d([0x7E])[0] == 448.0
    assert d([0x08])[0] == 2.0 ** -6
    assert d([0x01])[0] == 2.0 ** -9
    assert d([0x07])[0] == 7 * 2.0 ** -9
    assert d([0x38])[0] == 1.0
    assert d([0xB8])[0] == -1.0
    assert d([0x00])[0] == 0.0 and d([0x80])[0] == 0.0
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])


def test_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))


@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8_is_the_dense_oracle_on_dequantised_values(causal):
    rng = np.random.default_rng(8)
    n, d = 40, 16
    x = [torch.tensor(rng.standard_normal((n, d)) * 3, dtype=torch.float32).to(torch.float8_e4m3fn) for _ in range(3)]
    codes = [t.view(torch.uint8).numpy() for t in x]
    deq = [t.to(torch.float64).numpy() for t in x]
    scales = (0.5, 0.25, 2.0)
    o, lse = oracle.forward_fp8(*codes, *scales, 0.3, causal)
    o_ref, lse_ref = oracle.forward(deq[0] * 0.5, deq[1] * 0.25, deq[2] * 2.0, 0.3, causal)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)


def test_planted_bias_error_is_caught(monkeypatch):
    real = np.exp2
    monkeypatch.setattr(fp8_mod.np, "exp2", lambda x: real(np.asarray(x) - 1.0))
    try:
        assert fp8_mod.e4m3_decode([0x38])[0] != 1.0
    finally:
        monkeypatch.undo()
    assert fp8_mod.e4m3_decode([0x38])[0] == 1.0
