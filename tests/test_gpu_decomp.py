"""Parity of the mixed-precision decomposition path (sq_decomp_select,
sq_decomp_prepare_weights, sq_decomp_quant_act, sq_decomp_gemm) with the CPU
oracle, through the C ABI.

The oracle follows the pages literally (gather the bulk columns, quantise them,
integer matmul over the compacted K, add the binary32 outlier product); the
library keeps full-width int8 operands with the outlier columns zeroed.  Bar:
the chosen channels, codes (bulk columns equal to the oracle's, outlier columns
zero), scales and accumulators bit-exact; fp32 outputs bit-exact (within 1e-5
relative), bf16 outputs the RNE rounding of the oracle's fp32 (within 2^-8).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, assert_out_close, dev_act, host, misaligned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _keep(K, idx):
    return np.setdiff1d(np.arange(K), idx)


@pytest.mark.parametrize("K,n_o", [(1, 0), (1, 1), (83, 5), (8192, 41), (20000, 3), (300, 300)])
def test_decomp_select(sq, K, n_o):
    rng = np.random.default_rng(K + n_o)
    a = rng.uniform(0, 10, K).astype(np.float32)
    if K > 10:
        a[rng.choice(K, 6, replace=False)] = 7.5      # ties
    idx, mask = sq.sq_decomp_select(torch.from_numpy(a).to(DEV), n_o)
    want = O.decomp_select(a, n_o)
    assert np.array_equal(host(idx), want)
    m = np.ones(K, np.float32)
    m[want] = 0
    assert np.array_equal(host(mask), m)


def _prep_gpu(sq, X, xdt, W, n_o):
    a = O.col_absmax(X)
    idx, mask = sq.sq_decomp_select(torch.from_numpy(a).to(DEV), n_o)
    Wd = torch.from_numpy(W).to(DEV)
    Wq, ws, Wo = sq.sq_decomp_prepare_weights(Wd, mask, idx)
    return idx, mask, Wq, ws, Wo


def _check_split(Xq_g, xs_g, Xo_g, Xq_r, xs_r, Xo_r, idx):
    K = Xq_g.shape[1]
    keep = _keep(K, idx)
    assert np.array_equal(Xq_g[:, keep], Xq_r)
    assert not Xq_g[:, idx].any()
    assert np.array_equal(xs_g, xs_r)
    assert np.array_equal(Xo_g, Xo_r.T)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,K,n_o", [(1, 8, 16, 1), (16, 300, 512, 7), (70, 200, 1040, 4),
                                       (300, 520, 2048, 12), (33, 64, 133, 2), (129, 136, 256, 0),
                                       (40, 72, 256, 9), (5, 96, 1024, 250), (100, 12800, 512, 9),
                                       (200, 24576, 256, 9)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_decomp_layer(sq, xdt, T, N, K, n_o, out):
    rng = np.random.default_rng(T * 7 + N + K + n_o)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, rng.choice(K, min(K, 5), replace=False)] *= 30
    if xdt == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    idx, mask, Wq, ws, Wo = _prep_gpu(sq, X, xdt, W, n_o)
    idx_h = host(idx)
    Wq_r, ws_r, Wo_r = O.decomp_prepare(W, idx_h)
    _check_split(host(Wq), host(ws), host(Wo), Wq_r, ws_r, Wo_r, idx_h)
    Xd = dev_act(X, xdt)
    Xq, xs, Xo = sq.sq_decomp_quant_act(Xd, mask, idx)
    y_r, Xq_r, xs_r, Xo_r, acc_r = O.decomp_linear(X, idx_h, Wq_r, ws_r, Wo_r)
    _check_split(host(Xq), host(xs), host(Xo), Xq_r, xs_r, Xo_r, idx_h)
    ydt = torch.float32 if out == "f32" else torch.bfloat16
    y = sq.sq_decomp_gemm(Xq, xs, Wq, ws, Xo, Wo, out_dtype=ydt)
    assert_out_close(host(y), y_r, out)
    # the bulk accumulators alone are the plain GEMM's
    assert np.array_equal(host(sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.int32)), acc_r)
    if T * K > 16:
        Xq2, xs2, Xo2 = sq.sq_decomp_quant_act(misaligned(Xd), mask, idx)
        _check_split(host(Xq2), host(xs2), host(Xo2), Xq_r, xs_r, Xo_r, idx_h)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,K,n_o", [(100, 96, 512, 90), (100, 96, 512, 110), (2048, 2048, 256, 120),
                                       (4096, 4096, 128, 26), (4096, 4096, 128, 30),
                                       (16, 16390, 8192, 41), (5, 16384, 12288, 48), (9, 16448, 8192, 49)])
def test_decomp_gemm_outlier_staging(sq, T, N, K, n_o, out):
    """Prefill tiles copy their outlier operands into LDS when they fit (64x64
    tiles up to ~90 outliers, 128x128 up to ~94-107, 256x256 up to 26) and read
    them from global memory otherwise; the 1 KB-segment decode form takes up to
    48 outliers (staged in LDS), more go to the other decode form: outlier counts
    on both sides of those limits, outputs in full."""
    rng = np.random.default_rng(T + N + K + n_o)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, rng.choice(K, n_o, replace=False)] *= 25
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    idx, mask, Wq, ws, Wo = _prep_gpu(sq, X, "f32", W, n_o)
    idx_h = host(idx)
    Wq_r, ws_r, Wo_r = O.decomp_prepare(W, idx_h)
    Xq, xs, Xo = sq.sq_decomp_quant_act(dev_act(X, "f32"), mask, idx)
    y_r, *_ = O.decomp_linear(X, idx_h, Wq_r, ws_r, Wo_r)
    y = sq.sq_decomp_gemm(Xq, xs, Wq, ws, Xo, Wo, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    assert_out_close(host(y), y_r, out)


def test_decomp_generic_gemm_path(sq):
    """Misaligned int8 operands take the one-output-per-thread kernel."""
    rng = np.random.default_rng(5)
    T, N, K = 20, 36, 64
    X = rng.standard_normal((T, K)).astype(np.float32) * 3
    W = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    idx, mask, Wq, ws, Wo = _prep_gpu(sq, X, "f32", W, 3)
    Xq, xs, Xo = sq.sq_decomp_quant_act(dev_act(X, "f32"), mask, idx)
    y = sq.sq_decomp_gemm(misaligned(Xq), xs, misaligned(Wq), ws, Xo, Wo, out_dtype=torch.float32)
    idx_h = host(idx)
    Wq_r, ws_r, Wo_r = O.decomp_prepare(W, idx_h)
    y_r, *_ = O.decomp_linear(X, idx_h, Wq_r, ws_r, Wo_r)
    assert_out_close(host(y), y_r, "f32")


@pytest.mark.parametrize("name,n_o", [("decode_t16_k8192_n28672", 41), ("prefill_t2048_k4096_n16384", 8)])
def test_decomp_full_size(sq, name, n_o):
    """The decode and prefill workloads with their planted channel count taken as
    the static outlier set, chosen from the calibration draw: the chosen set,
    codes, scales, bulk accumulators and outputs, all in full."""
    w = WL.make(name)
    a = O.col_absmax(w.X_calib)
    idx, mask = sq.sq_decomp_select(torch.from_numpy(a).to(DEV), n_o)
    idx_h = host(idx)
    assert np.array_equal(idx_h, O.decomp_select(a, n_o))
    assert set(idx_h.tolist()) == set(np.asarray(w.outliers).tolist())
    Wq, ws, Wo = sq.sq_decomp_prepare_weights(torch.from_numpy(w.W).to(DEV), mask, idx)
    Wq_r, ws_r, Wo_r = O.decomp_prepare(w.W, idx_h)
    _check_split(host(Wq), host(ws), host(Wo), Wq_r, ws_r, Wo_r, idx_h)
    Xq, xs, Xo = sq.sq_decomp_quant_act(dev_act(w.X, w.x_dtype), mask, idx)
    Xb, Xo_r = O.decomp_split(w.X, idx_h)
    Xq_r, xs_r = O.quant_act(Xb, None)
    _check_split(host(Xq), host(xs), host(Xo), Xq_r, xs_r, Xo_r, idx_h)
    y = host(sq.sq_decomp_gemm(Xq, xs, Wq, ws, Xo, Wo, out_dtype=torch.bfloat16))
    y_r, _, _, _, acc_r = O.decomp_linear(w.X, idx_h, Wq_r, ws_r, Wo_r)
    assert np.array_equal(host(sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.int32)), acc_r)
    assert_out_close(y, y_r, "bf16")
