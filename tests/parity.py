"""Shared comparison helpers for the GPU parity tests (oracle vs HIP path).

Tolerances (written here once, used by every parity test):
  fp32 path:  max |x - x*| <= 1e-5 on O and lse.
  bf16 path:  |O - O*| <= 2e-2 + 2e-2 |O*| elementwise (the "2e-2 abs and 2e-2
              rel" bound read as the usual allclose rule, since a pure relative
              bound is meaningless where O* is near zero), |lse - lse*| <= 1e-3.
  gradients:  the same 2e-2 / 2e-2 rule on dq, dk, dv.
The method is exact only up to floating-point reassociation, so no floating
result is compared bitwise; index/count bookkeeping is (see test_bookkeeping).
"""

import numpy as np
import torch

F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 2e-2
LSE_ATOL = 1e-3
GRAD_ATOL, GRAD_RTOL = 2e-2, 2e-2


def host(t):
    """Exact host copy (bf16 and fp32 both widen exactly to fp32/fp64)."""
    return t.detach().to(torch.float32).cpu().numpy()


def allclose_report(x, ref, atol, rtol):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(x - ref)
    bound = atol + rtol * np.abs(ref)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    return dict(
        ok=bool(np.all(err <= bound)) and bool(np.all(np.isfinite(x))),
        max_abs=float(err.max()) if err.size else 0.0,
        max_rel=float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0,
        worst=tuple(int(i) for i in worst),
        worst_ratio=float(ratio.max()) if ratio.size else 0.0,
    )


def assert_close(x, ref, atol, rtol, what):
    r = allclose_report(x, ref, atol, rtol)
    assert r["ok"], f"{what}: max_abs={r['max_abs']:.3e} max_rel={r['max_rel']:.3e} worst index {r['worst']} (err/bound {r['worst_ratio']:.2f})"
    return r
