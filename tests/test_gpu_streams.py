"""Concurrent calls: two host threads, each with its own stream (default
priority), enqueue the run-time layer on different inputs at the same time; the
results equal those of the same calls made one after another."""
import threading

import numpy as np
import pytest
import torch

from gpu_util import DEV, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def test_two_threads_two_streams(sq):
    rng = np.random.default_rng(17)
    shapes = [(300, 384, 512), (16, 1024, 2048)]
    layers = []
    for T, N, K in shapes:
        X = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
        W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
        s, _, _ = sq.sq_smooth_scales(X, W, 0.5)
        Wq, ws = sq.sq_quantize_weights(W, s)
        layers.append((X, s, Wq, ws))
    torch.cuda.synchronize()
    want = [host(sq.sq_w8a8_linear(X, s, Wq, ws)) for X, s, Wq, ws in layers]
    torch.cuda.synchronize()

    reps = 20
    got = [[None] * reps for _ in layers]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(DEV)
            stream = torch.cuda.Stream()
            X, s, Wq, ws = layers[i]
            with torch.cuda.stream(stream):
                outs = [sq.sq_w8a8_linear(X, s, Wq, ws) for _ in range(reps)]
            stream.synchronize()
            for r, y in enumerate(outs):
                got[i][r] = host(y)
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(layers))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(len(layers)):
        for r in range(reps):
            assert np.array_equal(got[i][r], want[i]), f"layer {i} call {r}"
