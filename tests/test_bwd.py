"""GPU parity of the backward path (fa_backward) against the fp64 oracle's analytic gradients.

O and lse come from fa_forward on the same inputs; the oracle uses its own
fp64 O in D = rowsum(dO * O). For rows of moderate sharpness (the N(0, 1),
scale 1/sqrt(d) workloads) the bf16 rounding of the stored O stays well inside
the tolerance; for near one-hot rows it does not (see
test_backward_sharp_softmax_rows, which forms the oracle's D from its own O
rounded to bf16). dq, dk, dv must satisfy |x - x*| <= 2e-2 + 2e-2 |x*|.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import backward, backward_workspace_bytes, forward
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import GRAD_ATOL, GRAD_RTOL, assert_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _run(q, k, v, do, causal, scale, workspace=None):
    o, lse = forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=causal, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check(q, k, v, do, dq, dk, dv, causal, scale, heads):
    for b, h in heads:
        dq_ref, dk_ref, dv_ref, _, _ = oracle.backward(
            host(q[b, h]), host(k[b, h]), host(v[b, h]), host(do[b, h]), scale, causal
        )
        assert_close(host(dv[b, h]), dv_ref, GRAD_ATOL, GRAD_RTOL, f"dv head {(b, h)}")
        assert_close(host(dk[b, h]), dk_ref, GRAD_ATOL, GRAD_RTOL, f"dk head {(b, h)}")
        assert_close(host(dq[b, h]), dq_ref, GRAD_ATOL, GRAD_RTOL, f"dq head {(b, h)}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 257, 300, 513])
def test_backward_small_shapes(N, d, causal):
    _say("bwd sweep", N, d, causal)
    cfg = dict(dtype="bf16", seed=500 + 3 * N + d)
    B, H = 2, 2
    q, k, v, do = W.make_inputs(cfg, DEV, with_do=True, shape=(B, H, N, d))
    scale = 1 / math.sqrt(d)
    _, _, dq, dk, dv = _run(q, k, v, do, causal, scale)
    _check(q, k, v, do, dq, dk, dv, causal, scale, [(b, h) for b in range(B) for h in range(H)])


@pytest.mark.parametrize("B,H,N,d", [(2, 16, 700, 128), (4, 16, 300, 64)])
def test_backward_causal_heads_interleaved_on_each_xcd(B, H, N, d):
    """32 or 64 heads of 256-row query blocks: each XCD's share of the dQ grid
    is 4 or 8 whole heads, which the causal kernels issue longest block first
    across groups of 4 heads (the dK/dV kernel its 128-key blocks likewise).
    Every head's gradients are checked."""
    _say("bwd interleaved heads", B, H, N, d)
    cfg = dict(dtype="bf16", seed=900 + N + d)
    q, k, v, do = W.make_inputs(cfg, DEV, with_do=True, shape=(B, H, N, d))
    scale = 1 / math.sqrt(d)
    _, _, dq, dk, dv = _run(q, k, v, do, True, scale)
    _check(q, k, v, do, dq, dk, dv, True, scale, [(b, h) for b in range(B) for h in range(H)])


def test_backward_nondefault_scale():
    _say("bwd scale 0.05")
    q, k, v, do = W.make_inputs(dict(dtype="bf16", seed=78), DEV, with_do=True, shape=(1, 2, 333, 128))
    _, _, dq, dk, dv = _run(q, k, v, do, True, 0.05)
    _check(q, k, v, do, dq, dk, dv, True, 0.05, [(0, 0), (0, 1)])


U_BF16 = 2.0**-8  # unit roundoff of round-to-nearest-even bf16 (8 significant bits)


def bf16_first_order_bounds(q, k, v, do, scale, causal):
    """First-order error bounds, elementwise, for the bf16 roundings of the method's
    intermediates, derived from the arithmetic with the oracle's own P, O, dS:
      O stored as bf16 and P rounded to bf16 in the forward's P V product give
          |dO_err_i| <= u sum_k |dO_ik| (|O_ik| + sum_j P_ij |V_jk|)  =: e_D_i  (error of D_i)
      dS_ij = P_ij (dP_ij - D_i) then carries P_ij e_D_i, and is rounded to bf16
      before the dK and dQ products: |dS_err_ij| <= P_ij e_D_i + u |dS_ij|
      dV_j = sum_i bf16(P_ij) dO_i:        u sum_i P_ij |dO_i|
      dK_j = scale sum_i dS_ij q_i:        scale sum_i |dS_err_ij| |q_i|
      dQ_i = scale sum_j dS_ij k_j:        scale sum_j |dS_err_ij| |k_j|
    """
    u = U_BF16
    n = q.shape[0]
    q, k, v, do = (x.astype(np.float64) for x in (q, k, v, do))
    p, _ = oracle.softmax_rows(oracle.scores(q, k, scale, np.arange(n), causal))
    o = p @ v
    ds = p * ((do @ v.T) - np.sum(do * o, axis=1)[:, None])
    e_d = u * np.sum(np.abs(do) * (np.abs(o) + p @ np.abs(v)), axis=1)
    e_ds = p * e_d[:, None] + u * np.abs(ds)
    return {
        "dv": u * (p.T @ np.abs(do)),
        "dk": scale * (e_ds.T @ np.abs(q)),
        "dq": scale * (e_ds @ np.abs(k)),
    }


@pytest.mark.parametrize("q_mult,scale", [(4.0, 1 / math.sqrt(128)), (4.0, 0.3)])
def test_backward_sharp_softmax_rows(q_mult, scale):
    # Rows far sharper than the configured workloads (Q x 4; at scale 0.3 the
    # median row puts 96% of its weight on one key). There dS = P (dP - D)
    # cancels for the dominant key and the bf16 roundings of O, P and dS are
    # amplified past the plain 2e-2 / 2e-2 rule. The bound is that rule plus
    # twice the first-order rounding bounds of bf16_first_order_bounds().
    _say("bwd sharp rows", q_mult, scale)
    q, k, v, do = W.make_inputs(dict(dtype="bf16", seed=77, q_mult=q_mult), DEV, with_do=True,
                                shape=(1, 2, 333, 128))
    _, _, dq, dk, dv = _run(q, k, v, do, True, scale)
    for b, h in [(0, 0), (0, 1)]:
        qh, kh, vh, doh = host(q[b, h]), host(k[b, h]), host(v[b, h]), host(do[b, h])
        dq_ref, dk_ref, dv_ref, _, _ = oracle.backward(qh, kh, vh, doh, scale, True)
        extra = bf16_first_order_bounds(qh, kh, vh, doh, scale, True)
        for name, got, ref in (("dv", dv, dv_ref), ("dk", dk, dk_ref), ("dq", dq, dq_ref)):
            err = np.abs(host(got[b, h]) - ref)
            bound = GRAD_ATOL + GRAD_RTOL * np.abs(ref) + 2 * extra[name]
            assert np.all(err <= bound), f"{name} head {(b, h)}: worst err/bound {(err / bound).max():.2f}"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_rising_scores(causal):
    """Scores that climb by about 4 (log2 units) per 64 keys (the forward's
    fixed-reference pass reruns such blocks), so lse grows along the rows and
    the late keys dominate. O and lse come from the library's forward; the
    bound is the plain rule plus twice the first-order bf16 rounding bounds,
    as for the sharp rows above."""
    _say("bwd rising scores", causal)
    B, H, N, d = 1, 2, 777, 128
    g = torch.Generator().manual_seed(91 + causal)
    scale = 1 / math.sqrt(d)
    step = 4.0 / (scale * math.log2(math.e) * d)
    ramp = (torch.arange(N, dtype=torch.float32) / 64 * step).view(1, 1, N, 1)
    q = (torch.randn(B, H, N, d, generator=g) + 1.0).to(torch.bfloat16).to(DEV)
    k = (torch.randn(B, H, N, d, generator=g) + ramp).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    _, _, dq, dk, dv = _run(q, k, v, do, causal, scale)
    for b, h in [(0, 0), (0, 1)]:
        qh, kh, vh, doh = host(q[b, h]), host(k[b, h]), host(v[b, h]), host(do[b, h])
        dq_ref, dk_ref, dv_ref, _, _ = oracle.backward(qh, kh, vh, doh, scale, causal)
        extra = bf16_first_order_bounds(qh, kh, vh, doh, scale, causal)
        for name, got, ref in (("dv", dv, dv_ref), ("dk", dk, dk_ref), ("dq", dq, dq_ref)):
            err = np.abs(host(got[b, h]) - ref)
            bound = GRAD_ATOL + GRAD_RTOL * np.abs(ref) + 2 * extra[name]
            assert np.all(err <= bound), f"{name} head {(b, h)}: worst err/bound {(err / bound).max():.2f}"


def test_config5_sampled_heads():
    cfg = W.config(5)
    _say("config 5", cfg["name"])
    q, k, v, do = W.make_inputs(cfg, DEV, with_do=True)
    _, _, dq, dk, dv = _run(q, k, v, do, cfg["causal"], cfg["scale"])
    heads = W.sample_heads(cfg["B"], cfg["H"], 2, cfg["seed"] + 1)
    _check(q, k, v, do, dq, dk, dv, cfg["causal"], cfg["scale"], heads)


@pytest.mark.timeout(900)
def test_backward_at_headline_size_one_head():
    # the fwd+bwd pass bench.py times, B=8 H=32 N=16384 d=128 causal: one sampled head in full
    cfg = W.config(3)
    _say("config 3 backward", cfg["name"])
    q, k, v, do = W.make_inputs(cfg, DEV, with_do=True)
    _, _, dq, dk, dv = _run(q, k, v, do, True, cfg["scale"])
    heads = W.sample_heads(cfg["B"], cfg["H"], 1, cfg["seed"] + 3)
    _check(q, k, v, do, dq, dk, dv, True, cfg["scale"], heads)
    # every head: the key gradients of a softmax row sum to zero, and the value
    # gradients sum to the sum of the output gradients (see the oracle's pins)
    dv_sum = dv.float().sum(dim=2)
    do_sum = do.float().sum(dim=2)
    assert torch.allclose(dv_sum, do_sum, atol=1.0, rtol=2e-2)


def test_gradients_deterministic_and_workspace_contents_irrelevant():
    _say("bwd determinism")
    B, H, N, d = 2, 3, 1000, 128
    q, k, v, do = W.make_inputs(dict(dtype="bf16", seed=8), DEV, with_do=True, shape=(B, H, N, d))
    ws = torch.empty(backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # NaN pattern everywhere: the library must clear what it uses
    _, _, dq1, dk1, dv1 = _run(q, k, v, do, True, 1 / math.sqrt(d), workspace=ws)
    ws.fill_(0x7F)
    _, _, dq2, dk2, dv2 = _run(q, k, v, do, True, 1 / math.sqrt(d), workspace=ws)
    for name, a, b_ in (("dq", dq1, dq2), ("dk", dk1, dk2), ("dv", dv1, dv2)):
        diff = (a.view(torch.int16) != b_.view(torch.int16)).nonzero()
        assert diff.shape[0] == 0, (
            f"{name} differs between runs at {diff.shape[0]} elements, first (b, h, row, col): "
            f"{diff[:6].tolist()}; max abs {(a.float() - b_.float()).abs().max().item():.3e}"
        )
    _check(q, k, v, do, dq1, dk1, dv1, True, 1 / math.sqrt(d), [(0, 0), (1, 2)])


@pytest.mark.parametrize("kv_heads", [16, 4])
def test_gradients_bitwise_repeatable_over_many_workgroups(kv_heads):
    """The dK/dV kernel hands P from one wave to its partner through LDS and
    streams query tiles through a shared ring: at config 5's shape (B4 H16
    N4096; 512 workgroups in flight at once, in whatever interleaving the
    device picks) repeated runs must agree bit for bit, with shared K/V
    heads too."""
    _say("bwd repeatability", kv_heads)
    cfg = W.config(5)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    q, k, v, do = W.make_inputs(cfg, DEV, with_do=True, kv_heads=kv_heads)
    o, lse = forward(q, k, v, causal=True)
    first = backward(q, k, v, o, do, lse, causal=True)
    for rep in range(6):
        again = backward(q, k, v, o, do, lse, causal=True)
        for name, a_, b_ in zip(("dq", "dk", "dv"), first, again):
            assert torch.equal(a_, b_), f"{name} differs in repeat {rep}"


def test_backward_outputs_write_nothing_outside_their_bounds():
    _say("bwd guard bands")
    B, H, N, d = 1, 2, 301, 128
    q, k, v, do = W.make_inputs(dict(dtype="bf16", seed=9), DEV, with_do=True, shape=(B, H, N, d))
    o, lse = forward(q, k, v, causal=True)
    pad, n = 4096, B * H * N * d
    bufs = [torch.full((n + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    views = [b_[pad:pad + n].view(B, H, N, d) for b_ in bufs]
    nbytes = backward_workspace_bytes(B, H, N, d)
    wsbuf = torch.full((nbytes + 2 * pad,), 0x55, dtype=torch.uint8, device=DEV)
    ws = wsbuf[pad:pad + nbytes]
    from exact_tiled_attention_38_amd import _lib
    import ctypes

    rc = _lib.lib().fa_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        views[0].data_ptr(), views[1].data_ptr(), views[2].data_ptr(), ws.data_ptr(),
        B, H, N, d, 1, ctypes.c_float(1 / math.sqrt(d)),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
    )
    assert rc == 0, _lib.status_string(rc)
    torch.cuda.synchronize()
    for b_ in bufs:
        assert torch.all(b_[:pad] == -7.0) and torch.all(b_[pad + n:] == -7.0)
    assert torch.all(wsbuf[:pad] == 0x55) and torch.all(wsbuf[pad + nbytes:] == 0x55)
    _check(q, k, v, do, views[0], views[1], views[2], True, 1 / math.sqrt(d), [(0, 0), (0, 1)])
