"""Concurrent calls: four host threads, each on its own default-priority
stream, run forward + backward, the fp8 forward and decode on their own
inputs at the same time. The library keeps no state between calls (apart
from the allocation-free decode's scratch, not used here), so every result
must equal, bit for bit, the same calls run one after another on one
stream."""

import math
import threading

import pytest
import torch

from exact_tiled_attention_38_amd import backward, decode, forward, forward_fp8
from exact_tiled_attention_38_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(i):
    B, H, Hkv, N, d = 1 + i % 2, 4, 2 if i % 2 else 4, 300 + 97 * i, 128
    bf = W.make_inputs(dict(dtype="bf16", seed=9000 + i), DEV, with_do=True, shape=(B, H, N, d), kv_heads=Hkv)
    f8 = W.make_fp8_inputs(dict(seed=9100 + i), DEV, shape=(B, H, N, d), kv_heads=Hkv)
    dec = W.make_decode_inputs(dict(B=B, H=H, Hkv=Hkv, Nq=1 + i, Nk=3000 + 500 * i, d=d, seed=9200 + i), DEV)
    return bf, f8, dec


def _calls(bf, f8, dec):
    q, k, v, do = bf
    scale = 1 / math.sqrt(q.shape[-1])
    o, lse = forward(q, k, v, causal=True, scale=scale)
    grads = backward(q, k, v, o, do, lse, causal=True, scale=scale)
    (q8, k8, v8), f = f8
    o8, l8 = forward_fp8(q8, k8, v8, *f, causal=True, scale=scale)
    od, ld = decode(*dec, causal=True, scale=scale)
    return (o, lse, *grads, o8, l8, od, ld)


def test_threads_on_separate_streams_match_serial_calls():
    print("[case] 4 threads, 4 streams", flush=True)
    inputs = [_inputs(i) for i in range(4)]
    torch.cuda.synchronize()
    serial = [_calls(*x) for x in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in inputs]
    results, errors = [None] * len(inputs), []
    start = threading.Barrier(len(inputs))

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                start.wait()
                for _ in range(3):
                    results[i] = _calls(*inputs[i])
                streams[i].synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append((i, e))

    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(results, serial)):
        for j, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"thread {i}, output {j} differs from the serial call"
