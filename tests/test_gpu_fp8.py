"""Parity of the FP8 E4M3 variant (sq_quantize_weights_fp8, sq_quant_act_fp8,
sq_fp8_gemm) with the CPU oracle, through the C ABI.

Bar: E4M3 codes and scales bit-exact.  The GEMM accumulates exact E4M3 products
on the matrix cores at less than full binary32 precision when their magnitudes
differ widely, so on such data its accumulators are compared with the oracle's
exact (binary64) dot products within 2^-11 * sum_k |products|; outputs within
that bound times x_scale * w_scale plus one binary32 rounding (and the bf16
rounding, 2^-8 relative, for bf16 out).  The largest error measured on these
inputs is 2.7e-4 of sum |products| (100 x 12800 x 112: few, widely spread
products); from K = 4096 on it stays below 5e-5.  On codes whose partial sums
binary32 holds exactly the matrix cores are exact, and there every accumulator
is compared bit for bit (tile shapes and all five workload shapes), which is
what catches a dropped, repeated or misplaced piece of K.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_act, host, misaligned

pytestmark = pytest.mark.gpu
ACC_BOUND = 2.0 ** -11


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _case(seed, T, K, N, dtype):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)).astype(np.float32)
    if K > 4:
        X[:, rng.choice(K, 3, replace=False)] *= 40
    if dtype == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    s = rng.uniform(0.3, 4.0, K).astype(np.float32)
    return X, W, s


# K % 16 == 0 takes the decode kernel up to 32 tokens, and up to 64 on layers of
# at most 32 channels per CU or K >= 12288 (16, 32 or 64 tokens per block; 16, 32
# or 64 channels per workgroup); else 64x64 tiles
SHAPES = [(1, 8, 16), (16, 300, 512), (70, 200, 1040), (300, 520, 2048), (33, 64, 133), (257, 264, 4096),
          (24, 100, 2048), (32, 264, 1024), (64, 264, 1024), (5, 72, 8208), (48, 6200, 272), (9, 8200, 272),
          (24, 9000, 400), (20, 8180, 272), (40, 10240, 208), (16, 12300, 96),
          (9, 8192, 16384), (40, 6200, 16400), (9, 12300, 8208)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,K", SHAPES)
def test_fp8_quantisers(sq, dtype, T, N, K):
    X, W, s = _case(T + N + K, T, K, N, dtype)
    sd = torch.from_numpy(s).to(DEV)
    Xd = dev_act(X, dtype)
    Xq, xs = sq.sq_quant_act_fp8(Xd, sd)
    Xq_r, xs_r = O.quant_act_fp8(X, s)
    assert np.array_equal(host(xs), xs_r) and np.array_equal(host(Xq), Xq_r)
    Wr = torch.from_numpy(W).to(torch.bfloat16).float().numpy() if dtype == "bf16" else W
    Wd = dev_act(Wr, dtype)
    Wq, ws = sq.sq_quantize_weights_fp8(Wd, sd)
    Wq_r, ws_r = O.quantize_weights_fp8(Wr, s)
    assert np.array_equal(host(ws), ws_r) and np.array_equal(host(Wq), Wq_r)
    if T * K > 16:
        Xq2, xs2 = sq.sq_quant_act_fp8(misaligned(Xd), sd)
        assert np.array_equal(host(Xq2), Xq_r) and np.array_equal(host(xs2), xs_r)


def test_fp8_quantiser_zero_and_saturation(sq):
    X = np.zeros((3, 64), np.float32)
    X[1, 5] = -7.0
    X[2] = np.linspace(-3, 3, 64, dtype=np.float32)
    Xq, xs = sq.sq_quant_act_fp8(dev_act(X, "f32"))
    Xq_r, xs_r = O.quant_act_fp8(X, None)
    assert np.array_equal(host(Xq), Xq_r) and np.array_equal(host(xs), xs_r)
    assert host(xs)[0] == 1.0 and not host(Xq)[0].any() and host(Xq)[1, 5] == 0xFE


def _check_gemm(sq, Xq_r, xs_r, Wq_r, ws_r, ti=None, ni=None):
    """Accumulators (unit scales), fp32 and bf16 outputs at the (t, n) pairs
    given, or at every pair (then from the oracle's full-matrix exact dot)."""
    T, N = Xq_r.shape[0], Wq_r.shape[0]
    Xq = torch.from_numpy(Xq_r).to(DEV)
    Wq = torch.from_numpy(Wq_r).to(DEV)
    ones_t, ones_n = torch.ones(T, device=DEV), torch.ones(N, device=DEV)
    acc = host(sq.sq_fp8_gemm(Xq, ones_t, Wq, ones_n, out_dtype=torch.float32))
    y32 = host(sq.sq_fp8_gemm(Xq, torch.from_numpy(xs_r).to(DEV), Wq, torch.from_numpy(ws_r).to(DEV),
                              out_dtype=torch.float32))
    yb = host(sq.sq_fp8_gemm(Xq, torch.from_numpy(xs_r).to(DEV), Wq, torch.from_numpy(ws_r).to(DEV),
                             out_dtype=torch.bfloat16))
    if ti is None:
        exact, sab = O.fp8_dot(Xq_r, Wq_r)
        g, y32, yb = acc.astype(np.float64), y32, yb
        sc = (xs_r[:, None] * ws_r[None, :]).astype(np.float32).astype(np.float64)
    else:
        exact, sab = O.fp8_dot_at(Xq_r, Wq_r, ti, ni)
        g, y32, yb = acc[ti, ni].astype(np.float64), y32[ti, ni], yb[ti, ni]
        sc = (xs_r[ti] * ws_r[ni]).astype(np.float32).astype(np.float64)
    del acc
    ratio = np.abs(g - exact) / np.maximum(sab, 1e-300)
    assert np.all(np.abs(g - exact) <= ACC_BOUND * sab), ratio.max()
    y_exact = exact * sc
    tol = ACC_BOUND * sab * sc + 2.0 ** -23 * np.abs(y_exact) + 1e-37
    assert np.all(np.abs(y32 - y_exact) <= tol)
    ybf = O.widen_bf16(yb).astype(np.float64)
    assert np.all(np.abs(ybf - y_exact) <= tol + 2.0 ** -8 * np.abs(y_exact))
    return float(ratio.max())


@pytest.mark.parametrize("T,N,K", SHAPES + [(9, 16390, 8192)])   # + the 1 KB-segment decode form, ragged
def test_fp8_gemm_accuracy(sq, T, N, K):
    X, W, s = _case(3 * T + N + K, T, K, N, "f32")
    Xq_r, xs_r = O.quant_act_fp8(X, s)
    Wq_r, ws_r = O.quantize_weights_fp8(W, s)
    r = _check_gemm(sq, Xq_r, xs_r, Wq_r, ws_r)
    print(f"fp8 gemm {T}x{N}x{K}: max |acc - exact| / sum|p| = {r:.3g}")


# One, two and three K stages (with K tails) on every FP8 tile: 64x64 and 128x128
# (256-byte stages), 64x128 (128-byte stages) and the persistent 256x256 with 8
# waves (128-byte stages); every output compared.
@pytest.mark.parametrize("T,N,K", [(300, 520, 112), (300, 520, 336), (300, 520, 608),
                                   (1000, 4100, 208), (1000, 4100, 336), (1000, 4100, 608),
                                   (100, 12800, 112), (100, 12800, 208), (128, 16384, 336),
                                   (768, 16384, 208), (200, 24576, 336), (100, 24600, 208),
                                   (2100, 8200, 64), (2100, 8200, 208), (2100, 8200, 336)])
def test_fp8_gemm_stage_counts(sq, T, N, K):
    X, W, s = _case(5 * T + N + K, T, K, N, "f32")
    Xq_r, xs_r = O.quant_act_fp8(X, s)
    Wq_r, ws_r = O.quantize_weights_fp8(W, s)
    _check_gemm(sq, Xq_r, xs_r, Wq_r, ws_r)


def _narrow_codes(rng, r, k):
    """E4M3 codes of 0 and of +-1.0 .. +-1.875 (exponent field 7): every product
    is a multiple of 2^-6 below 4, so every partial sum of up to 2^16 of them
    needs at most 24 significant bits and binary32 holds it exactly."""
    pool = np.array([0x00] + list(range(0x38, 0x40)) + list(range(0xB8, 0xC0)), np.uint8)
    return rng.choice(pool, (r, k)).astype(np.uint8)


@pytest.mark.parametrize("T,N,K", SHAPES + [(300, 520, 112), (1000, 4100, 336), (100, 12800, 208),
                                            (128, 16384, 336), (768, 16384, 208), (200, 24576, 336),
                                            (2100, 8200, 336),
                                            # 1 KB-segment decode form
                                            (16, 16390, 8192), (3, 16384, 12288),
                                            # the five workload shapes, in the bench's configuration
                                            (128, 1024, 1024), (512, 4096, 4096), (16, 28672, 8192),
                                            (2048, 16384, 4096), (8192, 8192, 8192)])
def test_fp8_gemm_exact_on_narrow_codes(sq, T, N, K):
    """On codes whose products and partial sums binary32 holds exactly, the FP8
    matrix cores are exact, so every accumulator must equal the oracle's exact
    dot product bit for bit: a dropped, repeated or misplaced chunk of K, a
    transposed operand or a wrong tile index shows up in every affected output,
    whatever the rounding behaviour on wide-range data."""
    rng = np.random.default_rng(T * 7 + N * 3 + K)
    Xq_r, Wq_r = _narrow_codes(rng, T, K), _narrow_codes(rng, N, K)
    Xq, Wq = torch.from_numpy(Xq_r).to(DEV), torch.from_numpy(Wq_r).to(DEV)
    acc = host(sq.sq_fp8_gemm(Xq, torch.ones(T, device=DEV), Wq, torch.ones(N, device=DEV),
                              out_dtype=torch.float32))
    exact, _ = O.fp8_dot(Xq_r, Wq_r)
    bad = np.argwhere(acc.astype(np.float64) != exact)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at (t, n) = {bad[:4].tolist()}"


def test_fp8_gemm_misaligned_generic(sq):
    X, W, s = _case(9, 20, 64, 36, "f32")
    Xq_r, xs_r = O.quant_act_fp8(X, s)
    Wq_r, ws_r = O.quantize_weights_fp8(W, s)
    Xq = misaligned(torch.from_numpy(Xq_r).to(DEV))
    Wq = misaligned(torch.from_numpy(Wq_r).to(DEV))
    y = host(sq.sq_fp8_gemm(Xq, torch.from_numpy(xs_r).to(DEV), Wq, torch.from_numpy(ws_r).to(DEV),
                            out_dtype=torch.float32))
    ti, ni = np.repeat(np.arange(20), 36), np.tile(np.arange(36), 20)
    exact, sab = O.fp8_dot_at(Xq_r, Wq_r, ti, ni)
    sc = (xs_r[ti] * ws_r[ni]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(y[ti, ni] - exact * sc) <= 64 * 2.0 ** -24 * sab * sc + 2.0 ** -23 * np.abs(exact * sc))


@pytest.mark.parametrize("name", ["heavy_t8192_k8192_n8192", "prefill_t2048_k4096_n16384",
                                  "decode_t16_k8192_n28672", "page_t512_k4096_n4096", "tiny_t128_k1024_n1024"])
def test_fp8_full_size(sq, name):
    """The workload's smoothed operands in FP8: all codes and scales; every GEMM
    output against the exact dot products."""
    w = WL.make(name)
    Xs = w.X if w.X_calib is None else w.X_calib
    s = O.smooth_scales(O.col_absmax(Xs), O.col_absmax(w.W), w.alpha)
    sd = torch.from_numpy(s).to(DEV)
    Xq, xs = sq.sq_quant_act_fp8(dev_act(w.X, w.x_dtype), sd)
    Wq, ws = sq.sq_quantize_weights_fp8(torch.from_numpy(w.W).to(DEV), sd)
    Xq_r, xs_r = O.quant_act_fp8(w.X, s)
    Wq_r, ws_r = O.quantize_weights_fp8(w.W, s)
    assert np.array_equal(host(xs), xs_r) and np.array_equal(host(Xq), Xq_r)
    assert np.array_equal(host(ws), ws_r) and np.array_equal(host(Wq), Wq_r)
    r = _check_gemm(sq, Xq_r, xs_r, Wq_r, ws_r)
    print(f"fp8 gemm {name}: max |acc - exact| / sum|p| = {r:.3g}")
