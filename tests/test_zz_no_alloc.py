"""The no-allocation layer call (sq_w8a8_linear_noalloc) through the C ABI:
its outputs equal sq_w8a8_linear's (which takes a caller workspace) bit for
bit, on two calls in a row whose second input is smaller, so leftovers of the
first call in the shared scratch cannot leak into the second."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import DEV, dev_act, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _layer(sq, name, tokens=None):
    w = WL.make(name, tokens=tokens)
    Xs = dev_act(w.stats_source, w.x_dtype)
    W = torch.from_numpy(w.W).to(DEV)
    s, _, _ = sq.sq_smooth_scales(Xs, W, w.alpha)
    Wq, ws = sq.sq_quantize_weights(W, s)
    return w, dev_act(w.X, w.x_dtype), s, Wq, ws


@pytest.mark.parametrize("first,second", [
    (("prefill_t2048_k4096_n16384", None), ("decode_t16_k8192_n28672", None)),
    (("page_t512_k4096_n4096", None), ("page_t512_k4096_n4096", 37)),
    (("decode_t16_k8192_n28672", None), ("tiny_t128_k1024_n1024", 5)),
])
def test_noalloc_matches_workspace_call(sq, first, second):
    for name, tokens in (first, second):
        w, X, s, Wq, ws = _layer(sq, name, tokens)
        ydt = torch.bfloat16 if w.y_dtype == "bf16" else torch.float32
        y_ref = sq.sq_w8a8_linear(X, s, Wq, ws, out_dtype=ydt)
        Y = torch.full((w.T, w.N), 7.0, dtype=ydt, device=DEV)
        sq.sq_w8a8_linear_noalloc(X, s, Wq, ws, Y, out_dtype=ydt)
        assert np.array_equal(host(Y), host(y_ref)), (name, tokens)


def test_noalloc_too_large_is_refused(sq):
    """More codes than the scratch holds: SQ_ERR_SCRATCH, and Y is untouched."""
    T, K, N = 4097, 8192, 64
    X = torch.ones((T, K), dtype=torch.bfloat16, device=DEV)
    Wq = torch.ones((N, K), dtype=torch.int8, device=DEV)
    ws = torch.ones(N, device=DEV)
    Y = torch.zeros((T, N), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="SQ_ERR_SCRATCH"):
        sq.sq_w8a8_linear_noalloc(X, None, Wq, ws, Y)
    torch.cuda.synchronize()
    assert not Y.any().item()
    # the largest token count that fits at K = 8192 (codes + scales, each padded
    # to 256 bytes, exactly 32 MiB) still runs
    T2 = 4094
    assert sq.sq_w8a8_linear_workspace_size(T2, K) == sq.SQ_NOALLOC_SCRATCH_BYTES
    y_ref = sq.sq_w8a8_linear(X[:T2], None, Wq, ws)
    Y2 = torch.empty((T2, N), dtype=torch.bfloat16, device=DEV)
    sq.sq_w8a8_linear_noalloc(X[:T2], None, Wq, ws, Y2)
    assert np.array_equal(host(Y2), host(y_ref))
