"""GPU parity of decode (fa_decode) and of the partial-result merge (fa_merge)
against the fp64 oracle (oracle/decode.py).

Decode: queries are the last Nq positions of a sequence of Nk cached keys;
with the causal mask query i sees keys j <= Nk - Nq + i. O must meet the
bf16 rule of tests/parity.py and lse |err| <= 1e-3. The shapes cover one and
several 32-key tiles, ragged tails, splits that end mid-tile, several 32-row
query blocks (shared key/value heads times Nq > 32), and the 100,000-key
long-context length.
Merge: results over disjoint key sets, combined, must equal the result over
all keys; empty parts (lse = -inf) must weigh nothing.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_38_amd import decode, decode_workspace_bytes, merge
from exact_tiled_attention_38_amd import workloads as W
from tests.parity import BF16_ATOL, BF16_RTOL, LSE_ATOL, assert_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, H, Hkv, Nq, Nk, d, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    return r(B, H, Nq, d), r(B, Hkv, Nk, d), r(B, Hkv, Nk, d)


def _check(q, k, v, o, lse, causal, scale, batches=None):
    for b in range(q.shape[0]) if batches is None else batches:
        o_ref, lse_ref = oracle.forward_decode_heads(host(q[b]), host(k[b]), host(v[b]), scale, causal)
        assert_close(host(o[b]), o_ref, BF16_ATOL, BF16_RTOL, f"o batch {b}")
        assert_close(host(lse[b]), lse_ref, LSE_ATOL, 0.0, f"lse batch {b}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv,Nq", [(4, 4, 1), (8, 2, 1), (8, 1, 3), (32, 1, 2), (4, 4, 9)])
@pytest.mark.parametrize("Nk", [1, 31, 33, 100, 1000, 4133])
def test_decode_shapes(Nk, H, Hkv, Nq, d, causal):
    if causal and Nq > Nk:
        pytest.skip("causal decode needs Nq <= Nk")
    _say("decode", Nk, H, Hkv, Nq, d, causal)
    B = 2
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 4000 + Nk + 13 * H + Hkv + 7 * Nq + d + causal)
    scale = 1 / math.sqrt(d)
    o, lse = decode(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, causal, scale)


def test_decode_many_splits_long_context():
    """B1 H8 Nq1 over 100,000 keys d128 (many key splits), every head."""
    _say("decode long")
    B, H, Hkv, Nq, Nk, d = 1, 8, 8, 1, 100000, 128
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 4101)
    o, lse = decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, True, 1 / math.sqrt(d))


def test_decode_sharp_rows_and_scale():
    """Queries scaled up (near one-hot rows) and a non-default scale."""
    _say("decode sharp")
    B, H, Hkv, Nq, Nk, d = 2, 8, 2, 2, 3000, 128
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 4102)
    q = (q.float() * 4).to(torch.bfloat16)
    o, lse = decode(q, k, v, causal=True, scale=0.3)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, True, 0.3)


def test_decode_with_all_queries_is_the_causal_forward():
    _say("decode Nq == Nk")
    from exact_tiled_attention_38_amd import forward

    B, H, N, d = 1, 2, 300, 128
    q, k, v = _inputs(B, H, H, N, N, d, 4103)
    o, lse = decode(q, k, v, causal=True)
    o_f, lse_f = forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, True, 1 / math.sqrt(d))
    assert_close(host(o), host(o_f), BF16_ATOL, BF16_RTOL, "decode vs forward")
    assert_close(host(lse), host(lse_f), LSE_ATOL, 0.0, "decode lse vs forward")


def test_decode_deterministic_and_workspace_contents_irrelevant():
    _say("decode determinism")
    B, H, Hkv, Nq, Nk, d = 2, 16, 4, 1, 20000, 128
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 4104)
    nbytes = decode_workspace_bytes(B, H, Hkv, Nq, Nk, d)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    first = decode(q, k, v, causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(first[0].float()).all() and torch.isfinite(first[1]).all()
    for fill in (0.0, 1e30):
        ws.fill_(fill)
        again = decode(q, k, v, causal=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])


def test_decode_writes_nothing_outside_its_outputs():
    _say("decode guard bands")
    B, H, Hkv, Nq, Nk, d = 1, 8, 2, 3, 777, 64
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 4105)
    G = 4096
    ob = torch.full((G + B * H * Nq * d + G,), 7.0, dtype=torch.bfloat16, device=DEV)
    lb = torch.full((G + B * H * Nq + G,), 7.0, dtype=torch.float32, device=DEV)
    o = ob[G:G + B * H * Nq * d].view(B, H, Nq, d)
    l = lb[G:G + B * H * Nq].view(B, H, Nq)
    decode(q, k, v, causal=True, out=o, lse=l)
    torch.cuda.synchronize()
    assert bool((ob[:G] == 7).all()) and bool((ob[-G:] == 7).all())
    assert bool((lb[:G] == 7).all()) and bool((lb[-G:] == 7).all())
    _check(q, k, v, o, l, True, 1 / math.sqrt(d))


@pytest.mark.parametrize("d", [64, 128])
def test_merge_of_key_shards_is_the_whole(d):
    """Decode over key shards (non-causal), merged, against the oracle over all keys."""
    _say("merge shards", d)
    B, H, Nq, Nk = 2, 4, 5, 2500
    q, k, v = _inputs(B, H, H, Nq, Nk, d, 4200 + d)
    cuts = [0, 700, 701, 1900, Nk]
    parts = [decode(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), causal=False)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o_parts = torch.stack([o for o, _ in parts]).contiguous()
    l_parts = torch.stack([l for _, l in parts]).contiguous()
    o, lse = merge(o_parts, l_parts)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (B, H, Nq)
    _check(q, k, v, o, lse, False, 1 / math.sqrt(d))


def test_merge_against_oracle_merge_with_empty_parts():
    _say("merge oracle parts")
    rng = np.random.default_rng(4300)
    S, rows, d = 5, 333, 128
    o_parts = rng.standard_normal((S, rows, d))
    lse_parts = rng.standard_normal((S, rows)) * 3
    lse_parts[1, :50] = -np.inf          # a part that saw no key for these rows
    lse_parts[:, 60] = -np.inf           # a row that saw no key at all
    ob = torch.tensor(o_parts, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    lb = torch.tensor(lse_parts, dtype=torch.float32).to(DEV)
    o, lse = merge(ob, lb)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_partials(host(ob), host(lb))
    assert_close(host(o), o_ref, BF16_ATOL, BF16_RTOL, "merged o")
    finite = np.isfinite(lse_ref)
    assert_close(host(lse)[finite], lse_ref[finite], LSE_ATOL, 0.0, "merged lse")
    assert np.all(host(lse)[~finite] == -np.inf) and np.all(host(o)[60] == 0)


def test_binding_checks():
    q = torch.zeros(1, 6, 1, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="divide"):
        decode(q, k, k)
    q = torch.zeros(1, 4, 20, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="shape"):
        decode(q, k, k, causal=True)  # Nq > Nk with the causal mask


@pytest.mark.parametrize("kind", ["decode", "decode_gqa"])
def test_bench_workloads_sampled_heads(kind):
    """The decode workloads the benchmark times (B8 H32 Nk16384 d128, Nq 1;
    32 or 8 key/value heads): sampled query heads against the oracle."""
    cfg = W.DECODE_WORKLOADS[kind]
    _say("decode workload", cfg["name"])
    q, k, v = W.make_decode_inputs(cfg, DEV)
    scale = 1 / math.sqrt(cfg["d"])
    o, lse = decode(q, k, v, causal=cfg["causal"], scale=scale)
    torch.cuda.synchronize()
    g = cfg["H"] // cfg["Hkv"]
    for b, h in W.sample_heads(cfg["B"], cfg["H"], 6, cfg["seed"] + 2):
        o_ref, lse_ref = oracle.forward_decode(host(q[b, h]), host(k[b, h // g]), host(v[b, h // g]), scale,
                                               cfg["causal"])
        assert_close(host(o[b, h]), o_ref, BF16_ATOL, BF16_RTOL, f"o head {(b, h)}")
        assert_close(host(lse[b, h]), lse_ref, LSE_ATOL, 0.0, f"lse head {(b, h)}")
