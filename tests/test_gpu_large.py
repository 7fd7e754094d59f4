"""GEMMs whose int8 operands span more than 2^31 bytes: decode-shaped weights
(both decode forms), and prefill tokens or weights (the tiled kernel).  The host
splits them into launch slices so that every 32-bit buffer offset of a launch
holds (csrc/slices.h, checked as arithmetic on the CPU by test_launch_slices.py);
here the slices run on the GPU: accumulators and bf16 outputs next to the slice
boundary, at both ends and at random rows, against the oracle's exact integer
products (maitreyasuin.github.io "...01-one-outlier", section "Which scales
factor out, and why")."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, host

pytestmark = pytest.mark.gpu

K = 8192
# rows of one launch slice for 64-row tiles at this K: (rows + 64) * K <= 2^31
SLICE = ((2 ** 31 // K - 64) // 64) * 64
N = SLICE + 16400


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module")
def weights():
    g = torch.Generator(device=DEV)
    g.manual_seed(20261)
    Wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    ws = torch.rand(N, device=DEV, generator=g) * 1e-3 + 1e-4
    yield Wq, ws
    del Wq
    torch.cuda.empty_cache()


def _channels(rng):
    near = np.arange(SLICE - 70, SLICE + 70)
    ends = np.concatenate([np.arange(0, 70), np.arange(N - 70, N)])
    rand = rng.choice(N, 500, replace=False)
    return np.unique(np.concatenate([near, ends, rand]))


# 3 tokens: the 1 KB-segment form; 20 tokens: the 256-byte form (64-channel tiles)
@pytest.mark.parametrize("T", [3, 20])
def test_decode_gemm_beyond_2gib(sq, weights, T):
    assert N * K > 2 ** 31
    Wq, ws = weights
    g = torch.Generator(device=DEV)
    g.manual_seed(T)
    Xq = torch.randint(-127, 128, (T, K), dtype=torch.int8, device=DEV, generator=g)
    xs = torch.rand(T, device=DEV, generator=g) * 1e-2 + 1e-3
    acc = sq.sq_w8a8_gemm(Xq, None, Wq, None, out_dtype=torch.int32)
    y = sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.bfloat16)
    ch = _channels(np.random.default_rng(T))
    idx = torch.from_numpy(ch).to(DEV)
    Xq_h, xs_h = host(Xq), host(xs)
    Wsel, ws_sel = host(Wq.index_select(0, idx)), host(ws.index_select(0, idx))
    acc_r = O.int_gemm(Xq_h, Wsel)
    acc_g = host(acc.index_select(1, idx))
    assert np.array_equal(acc_g, acc_r)
    y_g = host(y.index_select(1, idx))
    assert np.array_equal(y_g, O.to_bf16(O.dequant(acc_r, xs_h, ws_sel)))


# the tiled prefill GEMM slices tokens and channels by 256-row tiles
SLICE256 = ((2 ** 31 // K - 256) // 256) * 256


def _rows(rng, n, cut):
    near = np.arange(cut - 70, cut + 70)
    ends = np.concatenate([np.arange(0, 70), np.arange(n - 70, n)])
    return np.unique(np.concatenate([near, ends, rng.choice(n, 400, replace=False)]))


@pytest.mark.parametrize("tokens_sliced", [True, False])
def test_prefill_gemm_beyond_2gib(sq, tokens_sliced):
    big, small = SLICE256 + 1000, 300
    T, Nn = (big, small) if tokens_sliced else (small, big)
    g = torch.Generator(device=DEV)
    g.manual_seed(7 if tokens_sliced else 8)
    Xq = torch.randint(-127, 128, (T, K), dtype=torch.int8, device=DEV, generator=g)
    Wq = torch.randint(-127, 128, (Nn, K), dtype=torch.int8, device=DEV, generator=g)
    xs = torch.rand(T, device=DEV, generator=g) * 1e-2 + 1e-3
    ws = torch.rand(Nn, device=DEV, generator=g) * 1e-3 + 1e-4
    acc = sq.sq_w8a8_gemm(Xq, None, Wq, None, out_dtype=torch.int32)
    y = sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(3)
    if tokens_sliced:
        ti = torch.from_numpy(_rows(rng, T, SLICE256)).to(DEV)
        Xs, xss = host(Xq.index_select(0, ti)), host(xs.index_select(0, ti))
        Ws, wss = host(Wq), host(ws)
        acc_g, y_g = host(acc.index_select(0, ti)), host(y.index_select(0, ti))
    else:
        ni = torch.from_numpy(_rows(rng, Nn, SLICE256)).to(DEV)
        Xs, xss = host(Xq), host(xs)
        Ws, wss = host(Wq.index_select(0, ni)), host(ws.index_select(0, ni))
        acc_g, y_g = host(acc.index_select(1, ni)), host(y.index_select(1, ni))
    acc_r = O.int_gemm(Xs, Ws)
    assert np.array_equal(acc_g, acc_r)
    assert np.array_equal(y_g, O.to_bf16(O.dequant(acc_r, xss, wss)))
    del Xq, Wq, acc, y
    torch.cuda.empty_cache()
