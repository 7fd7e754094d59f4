"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar (identical inputs on both sides, seeded from workloads/):
  * int8 codes, int32 accumulators, column maxima: bit-exact;
  * x_scale / w_scale: bit-exact given the same smoothing factors s (the oracle is
    fed the GPU's s); s itself within 1e-6 relative of the oracle's;
  * fp32 outputs within 1e-5 relative, bf16 outputs within 2^-8 relative of the
    oracle's fp32 output (and, since the epilogue order is fixed, equal to the
    oracle's own fp32 and bf16 values).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, assert_out_close, bf16_round, dev_act, host, misaligned  # noqa: F401

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


# ------------------------------------------------------------------ reductions
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(1, 1), (37, 80), (37, 83), (300, 1000), (1025, 8), (5000, 24)])
def test_col_absmax(sq, dtype, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    A = (rng.standard_normal((rows, cols)) * rng.uniform(0.1, 50, cols)).astype(np.float32)
    if dtype == "bf16":
        A = bf16_round(A)
    A[rows // 2, cols // 3] = -1000.0
    a = dev_act(A, dtype)
    got = host(sq.sq_col_absmax(a))
    assert np.array_equal(got, O.col_absmax(A))
    if rows > 2:   # running maximum over two calls equals the maximum over all rows
        m = sq.sq_col_absmax(a[: rows // 2].contiguous())
        sq.sq_col_absmax(a[rows // 2:].contiguous(), amax=m, accumulate=True)
        assert np.array_equal(host(m), O.col_absmax(A))
    assert np.array_equal(host(sq.sq_col_absmax(misaligned(a))), O.col_absmax(A))


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,K", [(1, 3, 8), (37, 300, 1000), (600, 5, 4096), (2050, 1100, 2056), (40, 60, 83)])
def test_smooth_scales_dtypes(sq, xdt, wdt, T, N, K):
    """Both column maxima (one fused launch when both operands have 16-byte rows,
    two launches otherwise) for every dtype pair and uneven T, N."""
    rng = np.random.default_rng(T + 3 * N + 7 * K)
    X = (rng.standard_normal((T, K)) * rng.uniform(0.1, 40, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X[T // 2, K // 3] = -900.0
    W[N - 1, K - 1] = 3.0
    if xdt == "bf16":
        X = bf16_round(X)
    if wdt == "bf16":
        W = bf16_round(W)
    Xd, Wd = dev_act(X, xdt), dev_act(W, wdt)
    s, xa, wa = sq.sq_smooth_scales(Xd, Wd, 0.5)
    xa_r, wa_r = O.col_absmax(X), O.col_absmax(W)
    assert np.array_equal(host(xa), xa_r) and np.array_equal(host(wa), wa_r)
    np.testing.assert_allclose(host(s), O.smooth_scales(xa_r, wa_r, 0.5), rtol=1e-6, atol=0)
    s2, xa2, wa2 = sq.sq_smooth_scales(misaligned(Xd), Wd, 0.5)     # two-launch path
    assert np.array_equal(host(xa2), xa_r) and np.array_equal(host(wa2), wa_r)


@pytest.mark.parametrize("xdt,wdt", [("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("T,N,K", [(1, 1, 8), (37, 300, 1000), (600, 5, 4096), (40, 60, 83), (70, 2100, 8192)])
@pytest.mark.parametrize("maxima", [(False, True), (True, False), (False, False)])
def test_smooth_scales_without_maxima_outputs(sq, xdt, wdt, T, N, K, maxima):
    """x_absmax and/or w_absmax passed as NULL: the same factors, bit for bit, as
    with both outputs (vector and scalar forms of the in-workgroup weight maxima,
    ragged K), and the oracle's within 1e-6; alpha 0 and 1 exactly."""
    rng = np.random.default_rng(T * 3 + N + K)
    X = (rng.standard_normal((T, K)) * rng.uniform(0.1, 40, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, K // 2] = 0.0                     # a zero weight column: the 1e-8 floor
    X[T // 2, K // 3] = -900.0
    if xdt == "bf16":
        X = bf16_round(X)
    if wdt == "bf16":
        W = bf16_round(W)
    Xd, Wd = dev_act(X, xdt), dev_act(W, wdt)
    for alpha in (0.0, 0.5, 1.0):
        s_ref, xa, wa = sq.sq_smooth_scales(Xd, Wd, alpha)
        s, xa2, wa2 = sq.sq_smooth_scales(Xd, Wd, alpha, maxima=maxima)
        assert np.array_equal(host(s), host(s_ref))
        if maxima[0]:
            assert np.array_equal(host(xa2), host(xa))
        if maxima[1]:
            assert np.array_equal(host(wa2), host(wa))
        s_r = O.smooth_scales(O.col_absmax(X), O.col_absmax(W), alpha)
        np.testing.assert_allclose(host(s), s_r, rtol=1e-6, atol=0)
        if alpha in (0.0, 1.0):
            assert np.array_equal(host(s), s_r)
        # the scalar kernels (misaligned rows) give the same bits
        s3, _, _ = sq.sq_smooth_scales(misaligned(Xd), misaligned(Wd), alpha, maxima=maxima)
        assert np.array_equal(host(s3), host(s_ref))


@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.5, 0.75, 1.0])
def test_smooth_scales(sq, alpha):
    w = WL.page_tiny_fixture(seed=3, T=50, N=70, K=96)
    X = dev_act(w.X, "f32")
    W = torch.from_numpy(w.W).to(DEV)
    W[:, 5] = 0.0          # zero weight column and zero activation column: 1e-8 floor
    X[:, 9] = 0.0
    s, xa, wa = sq.sq_smooth_scales(X, W, alpha)
    xa_r, wa_r = O.col_absmax(host(X)), O.col_absmax(host(W))
    assert np.array_equal(host(xa), xa_r) and np.array_equal(host(wa), wa_r)
    s_r = O.smooth_scales(xa_r, wa_r, alpha)
    s_g = host(s)
    if alpha in (0.0, 1.0):
        assert np.array_equal(s_g, s_r)
    np.testing.assert_allclose(s_g, s_r, rtol=1e-6, atol=0)
    s2 = sq.sq_smooth_scales_from_absmax(xa, wa, alpha)
    assert np.array_equal(host(s2), s_g)


def test_smooth_scales_full_range(sq):
    rng = np.random.default_rng(17)
    xa = np.exp(rng.uniform(-25, 10, 200000)).astype(np.float32)
    wa = np.exp(rng.uniform(-25, 5, 200000)).astype(np.float32)
    xa[:10] = 0
    wa[5:15] = 0
    for alpha in (0.1, 0.5, 0.85):
        s = sq.sq_smooth_scales_from_absmax(torch.from_numpy(xa).to(DEV), torch.from_numpy(wa).to(DEV), alpha)
        np.testing.assert_allclose(host(s), O.smooth_scales(xa, wa, alpha), rtol=1e-6, atol=0)


# ------------------------------------------------------------------ quantisers
# (800, 2056) and (1537, 2048): more rows than the row quantiser's 3 workgroups
# per CU (768 on 256 CUs), so workgroups walk 2-3 rows and their last prefetch
# past the final row re-reads row R - 1
QSHAPES = [(1, 8), (37, 80), (5, 83), (64, 4096), (17, 16384), (3, 20000), (300, 1032), (2, 1), (800, 2056),
           (1537, 2048)]


def _special_rows(X):
    X = X.copy()
    X[0] = 0.0                                   # all-zero row: scale 1, codes 0
    if X.shape[0] > 2 and X.shape[1] >= 8:
        X[1] = -0.0
        X[2, :] = 0.0
        X[2, :5] = [127.0, 0.5, 1.5, 2.5, -2.5]  # ties (scale 1 when s is None)
    return X


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_s", [False, True])
@pytest.mark.parametrize("T,K", QSHAPES)
def test_quant_act(sq, dtype, with_s, T, K):
    rng = np.random.default_rng(T * 131 + K)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40
    X = _special_rows(X)
    if dtype == "bf16":
        X = bf16_round(X)
    s = np.exp(rng.uniform(-3, 3, K)).astype(np.float32) if with_s else None
    x = dev_act(X, dtype)
    sd = torch.from_numpy(s).to(DEV) if with_s else None
    Xq, xs = sq.sq_quant_act(x, sd)
    Xq_r, xs_r = O.quant_act(X, s)
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)
    assert host(Xq).min() >= -127
    if T > 2 and K >= 8 and not with_s:
        assert host(Xq)[2, :5].tolist() == [127, 0, 2, 2, -2]
    # the unaligned (scalar) kernel gives the same bits
    Xq2, xs2 = sq.sq_quant_act(misaligned(x), sd)
    assert np.array_equal(host(Xq2), Xq_r) and np.array_equal(host(xs2), xs_r)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_s", [False, True])
@pytest.mark.parametrize("N,K", QSHAPES)
def test_quantize_weights(sq, dtype, with_s, N, K):
    rng = np.random.default_rng(N * 17 + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W = _special_rows(W)
    if dtype == "bf16":
        W = bf16_round(W)
    s = np.exp(rng.uniform(-3, 3, K)).astype(np.float32) if with_s else None
    w = dev_act(W, dtype)
    sd = torch.from_numpy(s).to(DEV) if with_s else None
    Wq, ws = sq.sq_quantize_weights(w, sd)
    Wq_r, ws_r = O.quantize_weights(W, s)
    assert np.array_equal(host(ws), ws_r)
    assert np.array_equal(host(Wq), Wq_r)
    Wq2, ws2 = sq.sq_quantize_weights(misaligned(w), sd)
    assert np.array_equal(host(Wq2), Wq_r) and np.array_equal(host(ws2), ws_r)


# ----------------------------------------------------------------------- GEMM
def _codes(rng, r, k):
    return rng.integers(-127, 128, (r, k), dtype=np.int8)


GEMM_SHAPES = [
    # decode kernel (T <= 32, or T <= 64 with K >= 12288 or at most 32 channels per
    # CU), else 64x64 tiles (33-64 tokens); 16, 32 and 64 channels per workgroup,
    # 2 and 4 K-split waves
    (1, 1, 16), (1, 40, 64), (5, 129, 80), (16, 1000, 256), (17, 77, 1040), (32, 300, 528), (33, 64, 48),
    (64, 300, 528), (48, 28672, 80), (33, 136, 12288), (64, 72, 12304), (40, 4100, 1040), (64, 6200, 528),
    (20, 6200, 272), (9, 8200, 272), (24, 9000, 400), (20, 8180, 272), (33, 8192, 208), (48, 10240, 208), (16, 12300, 96),
    (3, 8192, 16384), (20, 6200, 16400), (40, 8192, 16384), (5, 12300, 8192), (16, 16000, 8208),
    # decode kernel, 1 KB-segment form (<= 16 tokens, >= 64 channels per CU, K a
    # multiple of 4096 from 8192): ragged channel tail, 1 and 9 tokens, 3 segments per wave
    (16, 16390, 8192), (1, 16384, 12288), (9, 16448, 8192),
    # prefill kernel, 64x64 tiles (< 256 tiles of 128x128; 256-byte K stages), ragged
    # edges and K tails; one, two, three and more stages
    (65, 40, 16), (100, 129, 64), (300, 1000, 80), (100, 129, 304), (65, 40, 688), (257, 513, 1040),
    (512, 1024, 4096),
    # prefill kernel, 128x128 tiles (>= 256 of them, < 256 of 256x256; 256-byte K
    # stages), ragged edges and K tails; one, two, three and five stages
    (1000, 4100, 208), (1000, 4100, 272), (1000, 4100, 608), (1100, 4000, 1040),
    # prefill kernel, 64x128 tiles (65-128 tokens, at least 3/4 of the CUs' worth of
    # 64-channel tiles; 128-byte K stages), ragged edges and K tails; one, two,
    # three and six stages
    (100, 12800, 48), (100, 12800, 208), (128, 16384, 336), (65, 14336, 656),
    # 65-128 tokens on 3/4 of the CUs' worth of 128-channel tiles: 128x128 tiles
    (100, 24600, 208),
    # prefill kernel, 256x256 tiles one per workgroup (3/4 to 1 per CU) and 128x256
    # tiles (3/4 of the CUs or more), ragged edges and K tails
    (768, 16384, 208), (1000, 12300, 80), (200, 24576, 336), (300, 24600, 48),
    # prefill kernel, 256x256 tiles (more than 256 of them: the persistent form;
    # 128-byte K stages), ragged edges and K tails; one, two and three stages
    (2100, 8200, 48), (2048, 8192, 64), (2100, 8200, 208), (2048, 8448, 256), (2100, 8200, 336),
    # generic kernel (K % 16 != 0)
    (3, 5, 7), (70, 33, 83), (1, 1, 1),
]


@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_gemm_int32_accumulators(sq, T, N, K):
    rng = np.random.default_rng(T * 1_000_003 + N * 101 + K)
    Xq, Wq = _codes(rng, T, K), _codes(rng, N, K)
    acc = sq.sq_w8a8_gemm(torch.from_numpy(Xq).to(DEV), None, torch.from_numpy(Wq).to(DEV), None,
                          out_dtype=torch.int32)
    assert np.array_equal(host(acc), O.int_gemm(Xq, Wq))


def test_decode_shapes_assume_256_cus(sq):
    """The decode shapes above reach the 4- and 8-wave and 32-channel forms of the
    decode kernel only on a GPU with 256 compute units (the forms are chosen by
    how many workgroups fill the CUs); on another CU count they would silently
    test other forms, so that is reported here."""
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,K", [(1, 40, 64), (17, 77, 1040), (300, 1000, 80), (2100, 8200, 48),
                                   # decode forms: 8 K-split waves (12288 <= N < 16384,
                                   # K >= 8192, <= 16 tokens); 32 channels with 8 or 4
                                   # waves (K >= 16384, 6144 <= N <= 8192); 32 channels
                                   # with 2 waves (N = 8192, 17-64 tokens)
                                   (5, 12300, 8192), (16, 16000, 8208), (3, 8192, 16384),
                                   # 1 KB-segment decode form, ragged and whole
                                   (16, 16390, 8192), (7, 16448, 12288),
                                   (40, 8192, 16384), (20, 6200, 16400), (33, 8192, 208),
                                   (70, 33, 83), (64, 130, 64), (129, 257, 64), (1000, 4100, 272),
                                   (100, 129, 688), (1000, 4100, 608), (2100, 8200, 336),
                                   (100, 12800, 208), (65, 14336, 656), (768, 16384, 208),
                                   (200, 24576, 336)])
def test_gemm_epilogue(sq, out, T, N, K):
    rng = np.random.default_rng(T + N + K)
    Xq, Wq = _codes(rng, T, K), _codes(rng, N, K)
    xs = np.exp(rng.uniform(-8, 2, T)).astype(np.float32)
    ws = np.exp(rng.uniform(-12, -2, N)).astype(np.float32)
    y = sq.sq_w8a8_gemm(torch.from_numpy(Xq).to(DEV), torch.from_numpy(xs).to(DEV),
                        torch.from_numpy(Wq).to(DEV), torch.from_numpy(ws).to(DEV),
                        out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    y_r = O.dequant(O.int_gemm(Xq, Wq), xs, ws)
    assert_out_close(host(y), y_r, out)


def _bf16_edge_values():
    """binary32 values at the hard cases of rounding to bf16: exact ties with an
    even and an odd kept half, one ulp either side of a tie, subnormals, and the
    top of the range (the tie between the largest finite bf16 and infinity)."""
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF]
    exps = [1, 2, 20, 100, 126, 127, 128, 150, 200, 253, 254]
    bits = [(e << 23) | (h << 16) | lo for e in exps for h in (0x00, 0x01, 0x7E, 0x7F) for lo in lows]
    bits += [(h << 16) | lo for h in (0x00, 0x01, 0x40, 0x7F) for lo in lows[1:]]   # subnormals
    bits = np.array(bits, np.uint32)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


@pytest.mark.parametrize("T,N,K", [(16, 64, 64), (300, 1000, 64), (2100, 8200, 48)])
def test_gemm_bf16_rounding_edges(sq, T, N, K):
    """One-hot codes make every accumulator 1, so y = fl32(x_scale * w_scale); the
    scales put rounding ties, subnormals and overflow into the bf16 epilogue
    (decode kernel, 64x64 tiles, persistent 256x256 tiles)."""
    v = _bf16_edge_values()
    xs = np.resize(v, T).astype(np.float32)
    ws = np.resize(np.array([1.0, -1.0, 1.0 + 2.0 ** -9, 3.0, 2.0 ** -20, 0.7], np.float32), N)
    Xq = np.zeros((T, K), np.int8)
    Wq = np.zeros((N, K), np.int8)
    Xq[:, 0] = 1
    Wq[:, 0] = 1
    y = sq.sq_w8a8_gemm(torch.from_numpy(Xq).to(DEV), torch.from_numpy(xs).to(DEV),
                        torch.from_numpy(Wq).to(DEV), torch.from_numpy(ws).to(DEV), out_dtype=torch.bfloat16)
    y_r = O.dequant(np.ones((T, N), np.int32), xs, ws)
    assert np.array_equal(host(y), O.to_bf16(y_r))


def test_gemm_unaligned_output_row(sq):
    """N % 4 != 0: element stores on the edge, same values."""
    rng = np.random.default_rng(5)
    for T, N, K in ((300, 1001, 64), (20, 1001, 64)):
        Xq, Wq = _codes(rng, T, K), _codes(rng, N, K)
        xs = rng.uniform(0.01, 1, T).astype(np.float32)
        ws = rng.uniform(0.001, 0.1, N).astype(np.float32)
        y = sq.sq_w8a8_gemm(torch.from_numpy(Xq).to(DEV), torch.from_numpy(xs).to(DEV),
                            torch.from_numpy(Wq).to(DEV), torch.from_numpy(ws).to(DEV),
                            out_dtype=torch.bfloat16)
        assert_out_close(host(y), O.dequant(O.int_gemm(Xq, Wq), xs, ws), "bf16")


@pytest.mark.parametrize("T,K", [(2, 133136), (2, 133144), (80, 133136)])
def test_gemm_int32_extremes(sq, T, K):
    """|acc| up to 127^2 K at the largest K the contract allows (no overflow)."""
    Xq = np.full((T, K), 127, np.int8)
    Xq[1] = -127
    Wq = np.full((3, K), 127, np.int8)
    Wq[2] = -127
    acc = host(sq.sq_w8a8_gemm(torch.from_numpy(Xq).to(DEV), None, torch.from_numpy(Wq).to(DEV),
                               None, out_dtype=torch.int32))
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K and acc[0, 2] == -127 * 127 * K
    assert np.array_equal(acc, O.int_gemm(Xq, Wq))


# ------------------------------------------------------------ linear end to end
def _prepare_gpu(sq, w, alpha):
    Xs = dev_act(w.stats_source, w.x_dtype)
    W = torch.from_numpy(w.W).to(DEV)
    s, xa, wa = sq.sq_smooth_scales(Xs, W, alpha)
    Wq, ws = sq.sq_quantize_weights(W, s)
    return s, xa, wa, Wq, ws


def _check_prepare(w, alpha, s, xa, wa, Wq, ws):
    xa_r, wa_r = O.col_absmax(w.stats_source), O.col_absmax(w.W)
    assert np.array_equal(host(xa), xa_r) and np.array_equal(host(wa), wa_r)
    s_g = host(s)
    np.testing.assert_allclose(s_g, O.smooth_scales(xa_r, wa_r, alpha), rtol=1e-6, atol=0)
    Wq_r, ws_r = O.quantize_weights(w.W, s_g)     # oracle fed the GPU's factors
    assert np.array_equal(host(ws), ws_r)
    assert np.array_equal(host(Wq), Wq_r)
    return s_g, Wq_r, ws_r


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_linear_tiny_and_page(sq, alpha):
    for name in ("tiny_t128_k1024_n1024", "page_t512_k4096_n4096"):
        w = WL.make(name)
        if alpha not in w.alphas and name.startswith("tiny"):
            continue
        s, xa, wa, Wq, ws = _prepare_gpu(sq, w, alpha)
        s_g, Wq_r, ws_r = _check_prepare(w, alpha, s, xa, wa, Wq, ws)
        X = dev_act(w.X, w.x_dtype)
        y = sq.sq_w8a8_linear(X, s, Wq, ws, out_dtype=torch.float32)
        Xq, xs = sq.sq_quant_act(X, s)
        Xq_r, xs_r = O.quant_act(w.X, s_g)
        assert np.array_equal(host(Xq), Xq_r) and np.array_equal(host(xs), xs_r)
        acc = sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.int32)
        acc_r = O.int_gemm(Xq_r, Wq_r)
        assert np.array_equal(host(acc), acc_r)
        assert_out_close(host(y), O.dequant(acc_r, xs_r, ws_r), "f32")


@pytest.mark.parametrize("name", ["decode_t16_k8192_n28672", "prefill_t2048_k4096_n16384",
                                  "heavy_t8192_k8192_n8192"])
def test_linear_full_size(sq, name):
    """Full-size workloads in the configuration the benchmark times: codes,
    scales, every int32 accumulator and every bf16 output compared in full with
    the oracle (the heavy 8192^3 product is ~5.5e11 integer multiply-adds of the
    oracle's loop)."""
    w = WL.make(name)
    alpha = w.alpha
    s, xa, wa, Wq, ws = _prepare_gpu(sq, w, alpha)
    s_g, Wq_r, ws_r = _check_prepare(w, alpha, s, xa, wa, Wq, ws)
    X = dev_act(w.X, w.x_dtype)
    y = sq.sq_w8a8_linear(X, s, Wq, ws, out_dtype=torch.bfloat16)
    Xq, xs = sq.sq_quant_act(X, s)
    Xq_r, xs_r = O.quant_act(w.X, s_g)
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)
    yh = host(y)
    acc = host(sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.int32))
    acc_r = O.int_gemm(Xq_r, Wq_r)
    bad = np.argwhere(acc != acc_r)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at (t, n) = {bad[:4].tolist()}"
    del acc
    assert_out_close(yh, O.dequant(acc_r, xs_r, ws_r), "bf16")
    del acc_r
    # the W8A8 layer actually tracks the exact product (smoothing worked)
    rows = np.arange(0, w.T, max(1, w.T // 16))
    ye = O.exact_product(w.X[rows], w.W)
    err = np.linalg.norm(O.widen_bf16(yh[rows]) - ye) / np.linalg.norm(ye)
    assert err < 0.05, err


def test_linear_edge_cases(sq):
    """T = 1, N = 1, K = 16, zero activation rows, zero weight rows."""
    rng = np.random.default_rng(9)
    for T, N, K in ((1, 1, 16), (1, 300, 64), (70, 1, 32), (3, 5, 16)):
        X = rng.standard_normal((T, K)).astype(np.float32)
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        X[0] = 0.0
        W[0] = 0.0
        Xd, Wd = dev_act(X, "f32"), torch.from_numpy(W).to(DEV)
        s, xa, wa = sq.sq_smooth_scales(Xd, Wd, 0.5)
        Wq, ws = sq.sq_quantize_weights(Wd, s)
        y = sq.sq_w8a8_linear(Xd, s, Wq, ws, out_dtype=torch.float32)
        s_g = host(s)
        Wq_r, ws_r = O.quantize_weights(W, s_g)
        Xq_r, xs_r = O.quant_act(X, s_g)
        y_r = O.dequant(O.int_gemm(Xq_r, Wq_r), xs_r, ws_r)
        assert np.array_equal(host(Wq), Wq_r)
        assert_out_close(host(y), y_r, "f32")
        assert not host(y)[0].any() and not host(y)[:, 0].any()
