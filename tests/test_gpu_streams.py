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


def test_persistent_gemms_on_two_streams(sq):
    """Two persistent-form GEMMs (int8 and FP8, more 256x256 tiles than CUs) enqueued
    at the same time from two threads on two streams share the GPU; each result
    equals the same call made alone."""
    rng = np.random.default_rng(23)
    T, N, K = 2100, 8200, 256
    Xq = torch.from_numpy(rng.integers(-127, 128, (T, K), dtype=np.int8)).to(DEV)
    Wq = torch.from_numpy(rng.integers(-127, 128, (N, K), dtype=np.int8)).to(DEV)
    xs = torch.from_numpy(np.exp(rng.uniform(-8, 0, T)).astype(np.float32)).to(DEV)
    ws = torch.from_numpy(np.exp(rng.uniform(-10, -2, N)).astype(np.float32)).to(DEV)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).to(DEV)
    X = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(DEV)
    Wq8, ws8 = sq.sq_quantize_weights_fp8(W)
    Xq8, xs8 = sq.sq_quant_act_fp8(X)
    calls = [lambda: sq.sq_w8a8_gemm(Xq, xs, Wq, ws), lambda: sq.sq_fp8_gemm(Xq8, xs8, Wq8, ws8)]
    torch.cuda.synchronize()
    want = [host(c()) for c in calls]
    torch.cuda.synchronize()

    reps = 6
    got = [[None] * reps for _ in calls]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(DEV)
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                outs = [calls[i]() for _ in range(reps)]
            stream.synchronize()
            for r, y in enumerate(outs):
                got[i][r] = host(y)
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(len(calls)):
        for r in range(reps):
            assert np.array_equal(got[i][r], want[i]), f"call {i} repetition {r}"
