"""Pins of the CPU oracle to what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
printed value on a page (tests/golden/*), a closed form, an invariant, a textbook
or library routine, or brute force on tiny inputs.  A plausible slip in the oracle
(wrong axis, multiply instead of divide, dropped clamp, truncation instead of
round-half-even, swapped scale) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as WL
from conftest import read_golden


# ---------------------------------------------------------------- page 3 numbers
@pytest.fixture(scope="module")
def page3():
    X, W, cols = WL.page3_experiment_data()
    return X, W, cols


def _golden_page3():
    g = {}
    sweep = []
    for row in read_golden("page3_experiment.txt"):
        if row[0] == "sweep":
            sweep.append(tuple(float(v) for v in row[1:]))
        else:
            g[row[0]] = float(row[1])
    return g, sweep


def test_page3_error_before_after(page3):
    """inferenceinterviews.com page, "A strong answer": before 0.0949 after 0.0181."""
    X, W, _ = page3
    g, _ = _golden_page3()
    assert round(O.w8a8_relative_error(X, W, None), 4) == g["error_before"]
    assert round(O.w8a8_relative_error(X, W, 0.5), 4) == g["error_after_alpha_0.5"]


def test_page3_outlier_severity(page3):
    """Same page: largest channel max / median channel max = 73; 127/73 = 1.7."""
    X, _, _ = page3
    g, _ = _golden_page3()
    r = O.channel_max_over_median(X.astype(np.float32))
    assert round(r) == g["act_ratio_before"]
    assert round(127 / round(r), 1) == g["steps_left"]


def test_page3_alpha_sweep(page3):
    """Same page, alpha table: act and weight max/median and W8A8 error per alpha."""
    X, W, _ = page3
    _, sweep = _golden_page3()
    X32, W32 = X.astype(np.float32), W.astype(np.float32)
    xa, wa = O.col_absmax(X32), O.col_absmax(W32)
    for alpha, act_r, w_r, err_pct in sweep:
        s = O.smooth_scales(xa, wa, alpha)
        Xh = X32 / s          # smoothed activations (fp32, as the layer sees them)
        Wh = W32 * s
        assert round(O.channel_max_over_median(Xh), 1) == act_r, alpha
        assert round(O.channel_max_over_median(Wh), 1) == w_r, alpha
        assert round(100 * O.w8a8_relative_error(X, W, alpha), 1) == err_pct, alpha


def test_page3_qualitative_drop_only_inside(page3):
    """Smoothing helps at alpha in [0.25, 0.75] on the page data; the endpoints
    are not asserted to help (alpha = 1 is worse than no smoothing, as printed)."""
    X, W, _ = page3
    before = O.w8a8_relative_error(X, W, None)
    for a in (0.25, 0.5, 0.75):
        assert O.w8a8_relative_error(X, W, a) < before
    assert O.w8a8_relative_error(X, W, 1.0) > before


# ------------------------------------------------------------ worked example (P4)
def test_worked_example_p4():
    """mercemay.com page, "Why the per-tensor scale cannot fix it": amax 30 gives
    scale about 0.236; 0.01 -> code 0; 0.5 -> code 2."""
    rows = {r[0]: r[1:] for r in read_golden("worked_example_p4.txt") if r[0] != "code"}
    codes = [r[1:] for r in read_golden("worked_example_p4.txt") if r[0] == "code"]
    L = int(rows["length"][0])
    rng = np.random.default_rng(5)
    x = rng.uniform(-0.99, 0.99, size=L).astype(np.float32)
    x[17] = float(rows["amax"][0])
    probe = {}
    for i, (v, _) in enumerate(codes):
        x[100 + i] = float(v)
        probe[100 + i] = codes[i]
    Xq, xs = O.quant_act(x[None, :], None)
    assert round(float(xs[0]), int(rows["scale_decimals"][0])) == float(rows["scale_approx"][0])
    for i, (v, c) in probe.items():
        assert int(Xq[0, i]) == int(c), v
    assert Xq[0, 17] == 127


# ------------------------------------------------------------ quantizer (P5 rules)
def test_zero_rows_give_scale_one_and_zero_codes():
    """maitreyasuin page, "The four operations": an all-zero tensor gives codes 0
    and scale 1.0 (no 0/0)."""
    rules = {r[0]: r[1] for r in read_golden("quantizer_rules_p5.txt")}
    X = np.zeros((3, 40), np.float32)
    X[1, 5] = 2.0
    Xq, xs = O.quant_act(X, None)
    assert xs[0] == float(rules["zero_scale"]) and xs[2] == float(rules["zero_scale"])
    assert not Xq[0].any() and not Xq[2].any()
    Wq, ws = O.quantize_weights(X, None)
    assert ws[0] == 1.0 and not Wq[0].any()
    # with smoothing, a zero row stays zero
    s = np.linspace(0.5, 3, 40).astype(np.float32)
    Xq, xs = O.quant_act(X, s)
    assert xs[0] == 1.0 and not Xq[0].any()


def test_round_half_even_ties():
    """Ties go to even (np.round / torch.round semantics used on the pages).  A row
    with amax 127 has scale exactly 1, so x/scale is x itself."""
    vals = [127.0, 0.5, 1.5, 2.5, -2.5, -0.5, 3.5, 126.5, -126.5, 0.49999997, 2.5000002]
    want = [127, 0, 2, 2, -2, 0, 4, 126, -126, 0, 3]
    X = np.array([vals], np.float32)
    Xq, xs = O.quant_act(X, None)
    assert xs[0] == 1.0
    assert Xq[0].tolist() == want
    Wq, ws = O.quantize_weights(X, None)
    assert ws[0] == 1.0 and Wq[0].tolist() == want


def test_code_range_and_full_scale():
    """Codes stay in [-127, 127] (never -128), and every nonzero row reaches
    |code| = 127 exactly at its absmax element."""
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    X[3] = -X[3]
    s = rng.uniform(0.1, 10, 300).astype(np.float32)
    for Xq, _ in (O.quant_act(X, s), O.quantize_weights(X, s)):
        assert Xq.min() >= -127 and Xq.max() <= 127
        assert (np.abs(Xq.astype(np.int32)).max(axis=1) == 127).all()
    Xq, _ = O.quant_act(X, s)
    am = np.argmax(np.abs(X / s), axis=1)
    assert (np.abs(Xq[np.arange(64), am]) == 127).all()


def test_round_trip_error_within_half_step():
    """x_hat = s q ("The four operations") is within half a step of x for every
    element, and the sign is kept: pins division by the scale (not
    multiplication) and nearest rounding (not truncation)."""
    rng = np.random.default_rng(12)
    X = (rng.standard_normal((50, 257)) * 3).astype(np.float32)
    s = rng.uniform(0.2, 5, 257).astype(np.float32)
    Xq, xs = O.quant_act(X, s)
    Xh = X.astype(np.float64) / s.astype(np.float64)
    deq = Xq.astype(np.float64) * xs[:, None].astype(np.float64)
    step = xs[:, None].astype(np.float64)
    assert (np.abs(deq - Xh) <= 0.5 * step * (1 + 1e-5)).all()
    assert (np.sign(Xq) * np.sign(Xh) >= 0).all()
    # nearest rounding leaves a quarter step on average; truncation half a step
    assert np.mean(np.abs(deq - Xh) / step) < 0.3
    # weights: the smoothing factor multiplies (W diag(s))
    Wq, ws = O.quantize_weights(X, s)
    Wh = X.astype(np.float64) * s.astype(np.float64)
    deqw = Wq.astype(np.float64) * ws[:, None].astype(np.float64)
    assert (np.abs(deqw - Wh) <= 0.5 * ws[:, None] * (1 + 1e-5)).all()


def test_scale_is_amax_over_127():
    """scale = limit / n with n = 127 ("The four operations")."""
    X = np.array([[0.0, -30.0, 3.0, 1.0], [254.0, 1.0, 2.0, -1.0]], np.float32)
    _, xs = O.quant_act(X, None)
    assert xs[0] == np.float32(30.0) / np.float32(127.0)
    assert xs[1] == np.float32(2.0)


# ----------------------------------------------------------- smoothing factors
def test_alpha_closed_forms():
    """multigrid.ai page, "Alpha: how much difficulty to move": alpha = 0 gives
    s = 1 / max|W_j|; alpha = 1 gives s = max|X_j|."""
    rng = np.random.default_rng(3)
    xa = rng.uniform(0.01, 200, 999).astype(np.float32)
    wa = rng.uniform(1e-3, 2, 999).astype(np.float32)
    s0 = O.smooth_scales(xa, wa, 0.0)
    s1 = O.smooth_scales(xa, wa, 1.0)
    assert np.array_equal(s1, xa)
    assert np.array_equal(s0, (np.float32(1.0) / wa).astype(np.float32))


def test_alpha_half_balances_maxima():
    """alpha = 0.5 is the geometric balance: after smoothing, each channel's
    activation max equals its weight max (maitreyasuin page, "Route it, or move
    it": both maxima become 3.86); for any alpha the product of the two maxima is
    unchanged, and s_j is monotone in alpha towards the activation side."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((200, 64)).astype(np.float32)
    X[:, [3, 40]] *= 50
    W = (rng.standard_normal((90, 64)) * 0.02).astype(np.float32)
    xa, wa = O.col_absmax(X), O.col_absmax(W)
    s = O.smooth_scales(xa, wa, 0.5)
    xh = np.abs(X / s).max(0)
    wh = np.abs(W * s).max(0)
    np.testing.assert_allclose(xh, wh, rtol=1e-6)
    for a in (0.0, 0.3, 0.75, 1.0):
        s = O.smooth_scales(xa, wa, a)
        np.testing.assert_allclose(np.abs(X / s).max(0) * np.abs(W * s).max(0),
                                   xa.astype(np.float64) * wa, rtol=1e-6)
    ratio = xa.astype(np.float64) * wa
    s_lo, s_hi = O.smooth_scales(xa, wa, 0.25), O.smooth_scales(xa, wa, 0.75)
    # d log s / d alpha = log(xa * wa): s grows with alpha exactly where xa*wa > 1
    clear = np.abs(np.log(ratio)) > 1e-3
    assert np.array_equal((s_hi > s_lo)[clear], (ratio > 1)[clear])


def test_smoothing_eps_clamp():
    """maitreyasuin page, "Route it, or move it": both maxima clamped below at
    1e-8 before the powers, so zero columns give finite factors."""
    xa = np.array([0.0, 0.0, 2.0], np.float32)
    wa = np.array([0.0, 4.0, 0.0], np.float32)
    eps = np.float32(1e-8)
    assert np.array_equal(O.smooth_scales(xa, wa, 1.0), np.array([eps, eps, 2.0], np.float32))
    s0 = O.smooth_scales(xa, wa, 0.0)
    assert s0[0] == np.float32(1.0 / np.float64(eps)) and s0[1] == np.float32(0.25)
    assert np.isfinite(O.smooth_scales(xa, wa, 0.5)).all()


def test_col_absmax_brute_force():
    """Column absmax against a plain loop and numpy's reduction."""
    rng = np.random.default_rng(9)
    A = rng.standard_normal((13, 7)).astype(np.float32)
    A[4, 2] = -99.0
    got = O.col_absmax(A)
    want = [max(abs(float(A[i, j])) for i in range(13)) for j in range(7)]
    assert got.tolist() == want
    assert np.array_equal(got, np.abs(A).max(axis=0))


def test_smoothing_identity_fp64():
    """XW^T = (X diag(s)^-1)(W diag(s))^T exactly over the reals (inferenceinterviews
    page, "What SmoothQuant does"; maitreyasuin page, "Route it, or move it"); in
    fp64 the relative difference is at rounding level (<= 1e-12), with the
    oracle's factors applied on the column (input-channel) axis."""
    w = WL.make("tiny_t128_k1024_n1024")
    xa, wa = O.col_absmax(w.X), O.col_absmax(w.W)
    s = O.smooth_scales(xa, wa, 0.5).astype(np.float64)
    X, W = w.X.astype(np.float64), w.W.astype(np.float64)
    Y = X @ W.T
    Ys = (X / s) @ (W * s).T
    assert np.linalg.norm(Ys - Y) / np.linalg.norm(Y) <= 1e-12
    # a factor applied on the wrong axis does not cancel
    bad = (X / s) @ W.T
    assert np.linalg.norm(bad - Y) / np.linalg.norm(Y) > 1e-2


def test_quantized_pipeline_tracks_smoothed_operands():
    """With the oracle's own quantizers, the dequantised smoothed operands
    multiply back to XW^T (orientation of s on both sides is right)."""
    w = WL.make("tiny_t128_k1024_n1024")
    p = O.prepare(w.X, w.W, 0.5)
    y, Xq, xs, acc = O.w8a8_linear(w.X, p["s"], p["Wq"], p["w_scale"])
    Y = O.exact_product(w.X, w.W)
    assert np.linalg.norm(y - Y) / np.linalg.norm(Y) < 0.03


# -------------------------------------------------------------- integer GEMM
@pytest.mark.parametrize("T,N,K", [(1, 1, 1), (3, 17, 64), (17, 3, 17), (64, 5, 3), (4, 64, 1)])
def test_int_gemm_brute_force(T, N, K):
    """acc_tn = sum_k P_tk Q_nk: pure-Python triple loop and an fp64 BLAS product
    (exact while |acc| < 2^53) agree with the oracle."""
    rng = np.random.default_rng(T * 1000 + N * 10 + K)
    Xq = rng.integers(-127, 128, (T, K), dtype=np.int8)
    Wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = O.int_gemm(Xq, Wq)
    for t in range(T):
        for n in range(N):
            assert acc[t, n] == sum(int(Xq[t, k]) * int(Wq[n, k]) for k in range(K))
    assert np.array_equal(acc, (Xq.astype(np.float64) @ Wq.astype(np.float64).T).astype(np.int64))
    ti = rng.integers(0, T, 9)
    ni = rng.integers(0, N, 9)
    assert np.array_equal(O.int_gemm_at(Xq, Wq, ti, ni), acc[ti, ni])


def test_int_gemm_extremes_and_overflow():
    """|acc| <= 127^2 K fits int32 up to K = 133144; one more overflows."""
    K = 133144
    Xq = np.full((1, K), 127, np.int8)
    Wq = np.full((2, K), 127, np.int8)
    Wq[1] = -127
    acc = O.int_gemm(Xq, Wq)
    assert acc[0, 0] == 127 * 127 * K and acc[0, 1] == -127 * 127 * K
    Xq2 = np.full((1, K + 1), 127, np.int8)
    with pytest.raises(OverflowError):
        O.int_gemm(Xq2, np.full((1, K + 1), 127, np.int8))


# ------------------------------------------------------------------ epilogue
def test_epilogue_factors_out():
    """maitreyasuin page, "Which scales factor out, and why": per-token and
    per-output-channel scales come out of the sum, so acc * (a_t * s_n) equals the
    fp64 product of the dequantised operands up to the two fp32 roundings of the
    epilogue (<= 2^-23 relative)."""
    rng = np.random.default_rng(21)
    Xq = rng.integers(-127, 128, (31, 70), dtype=np.int8)
    Wq = rng.integers(-127, 128, (23, 70), dtype=np.int8)
    xs = rng.uniform(0.001, 2, 31).astype(np.float32)
    ws = rng.uniform(0.0001, 0.1, 23).astype(np.float32)
    y = O.dequant(O.int_gemm(Xq, Wq), xs, ws).astype(np.float64)
    ref = (Xq * xs[:, None].astype(np.float64)) @ (Wq * ws[:, None].astype(np.float64)).T
    np.testing.assert_allclose(y, ref, rtol=2 ** -22, atol=0)
    # swapping the two scale vectors' roles breaks it
    bad = O.dequant(O.int_gemm(Xq, Wq)[:23, :23], ws, xs[:23]).astype(np.float64)
    assert not np.allclose(bad, ref[:23, :23], rtol=1e-3)
    yat = O.dequant_at(O.int_gemm(Xq, Wq)[[0, 5], [1, 7]], xs, ws, [0, 5], [1, 7])
    assert np.array_equal(yat, y[[0, 5], [1, 7]].astype(np.float32))


def test_epilogue_order_is_product_of_scales_first():
    """The epilogue multiplies by (sx * sw) formed first ("integer matmul, float
    epilogue" on the mercemay page); for a case where the two orders round apart
    the oracle takes this one."""
    rng = np.random.default_rng(8)
    acc = rng.integers(-2 ** 24, 2 ** 24, (1, 4000)).astype(np.int32)
    xs = np.array([0.1], np.float32)
    ws = rng.uniform(1e-3, 1, 4000).astype(np.float32)
    y = O.dequant(acc, xs, ws)[0]
    first = acc[0].astype(np.float32) * (xs[0] * ws)
    assert np.array_equal(y, first.astype(np.float32))
    other = (acc[0].astype(np.float32) * xs[0]) * ws
    assert not np.array_equal(y, other)


def test_bf16_rounding():
    """float32 -> bf16 nearest-even against torch's conversion, plus hand cases."""
    import torch
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    hand = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20, 0.0, -0.0],
                    np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81, 0x0000, 0x8000]
    assert O.to_bf16(hand).tolist() == want
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.to_bf16(y), ref)


# -------------------------------------------------------- qualitative drop
@pytest.mark.parametrize("name,tokens,alpha", [("tiny_t128_k1024_n1024", None, 0.5),
                                               ("page_t512_k4096_n4096", 128, 0.5)])
def test_smoothing_lowers_error_on_outlier_data(name, tokens, alpha):
    """W8A8 error after smoothing is below the error without it on outlier data
    (inferenceinterviews page: 9.5% -> 1.8%)."""
    w = WL.make(name, tokens=tokens)
    W = w.W if tokens is None else w.W[:1024]
    before = O.w8a8_relative_error(w.X, W, None)
    after = O.w8a8_relative_error(w.X, W, alpha)
    assert after < 0.5 * before


def test_smoothing_lowers_error_heavy_outliers():
    """Heavy-outlier structure (30% of channels x10..x60, alpha 0.75) at a reduced
    size: smoothing still lowers the error."""
    w = WL.make_linear(256, 512, 2048, n_out=614, mult_range=(10., 60.), seed=99)
    before = O.w8a8_relative_error(w.X, w.W, None)
    after = O.w8a8_relative_error(w.X, w.W, 0.75)
    assert after < before


def test_oracle_threads_independent():
    """Results do not depend on the OpenMP thread count (max and integer sums are
    order-free; each row is independent)."""
    w = WL.page_tiny_fixture()
    p = O.prepare(w.X, w.W, 0.5)
    y1 = O.w8a8_linear(w.X, p["s"], p["Wq"], p["w_scale"])[0]
    O.set_threads(1)
    try:
        y2 = O.w8a8_linear(w.X, p["s"], p["Wq"], p["w_scale"])[0]
    finally:
        O.set_threads(8)
    assert np.array_equal(y1, y2)
    assert math.isfinite(float(np.abs(y1).max()))


# ------------------------------------------- per-tensor activation scales (O2 / O3)
def test_page3_per_tensor_scales(page3):
    """inferenceinterviews.com page, "A strong answer" (formats paragraph): with
    per-tensor activation scales the same data gives 21% before, 2.9% after."""
    X, W, _ = page3
    g = {r[0]: float(r[1]) for r in read_golden("page3_per_tensor.txt")}
    assert round(100 * O.w8a8_relative_error(X, W, None, act="tensor")) == g["error_before_percent"]
    assert round(100 * O.w8a8_relative_error(X, W, 0.5, act="tensor"), 1) == \
        g["error_after_alpha_0.5_percent"]


def test_static_range_edge_127_6():
    """maitreyasuin page, "The four operations": with a range fixed in advance a
    value can land at 127.6 steps, which rounds to 128; clamped it is 127, never
    the int8 wrap -128.  clip = 127 gives scale exactly 1."""
    rules = {r[0]: r[1] for r in read_golden("quantizer_rules_p5.txt")}
    edge = float(rules["edge_value"])
    X = np.array([[edge, -edge, 128.4, 500.0, -1e4, 126.5, 0.5, -0.5, 1.5]], np.float32)
    Xq, xs = O.quant_act_static(X, None, 127.0)
    assert xs[0] == 1.0
    assert Xq[0, 0] == int(rules["edge_clamped"]) and Xq[0, 1] == -int(rules["edge_clamped"])
    assert Xq[0].tolist() == [127, -127, 127, 127, -127, 126, 0, 0, 2]
    assert int(Xq.min()) >= -127


def test_per_tensor_one_token_is_per_token():
    """With one token the tensor is the token: per-tensor dynamic quantisation
    must give exactly the per-token codes and scale (pinned separately)."""
    rng = np.random.default_rng(21)
    s = rng.uniform(0.2, 5, 777).astype(np.float32)
    for _ in range(5):
        x = (rng.standard_normal((1, 777)) * rng.uniform(0.1, 50)).astype(np.float32)
        q1, s1 = O.quant_act(x, s)
        q2, s2, amax = O.quant_act_per_tensor(x, s)
        assert s1[0] == s2[0] and np.array_equal(q1, q2)
        assert amax == np.max(np.abs(x[0] / s))


def test_per_tensor_scale_is_largest_token_scale():
    """amax over the tensor is the largest per-token amax, and fl32(a / 127) is
    monotone in a, so the tensor scale equals the largest per-token scale; the
    token that holds the maximum gets its per-token codes unchanged."""
    rng = np.random.default_rng(22)
    X = rng.standard_normal((40, 300)).astype(np.float32)
    X[:, rng.choice(300, 3, replace=False)] *= 40
    X[17] *= 3
    s = rng.uniform(0.5, 2, 300).astype(np.float32)
    qt, st = O.quant_act(X, s)
    qT, sT, amax = O.quant_act_per_tensor(X, s)
    assert np.all(sT == st.max())
    t = int(np.argmax(st))
    assert np.array_equal(qT[t], qt[t])
    # every other token is on a coarser grid: its codes shrink in magnitude
    assert np.all(np.abs(qT.astype(int)) <= np.abs(qt.astype(int)) + 1)


def test_per_tensor_absmax_planted():
    """The range is the largest |X_tk / s_k|: a planted value decides it."""
    X = np.zeros((9, 33), np.float32)
    X[3, 7] = -5.0
    X[8, 30] = 9.0
    s = np.ones(33, np.float32)
    s[7] = 0.5        # -5 / 0.5 = -10 -> 10 wins over 9 / 1
    assert O.act_tensor_absmax(X, s) == np.float32(10.0)
    assert O.act_tensor_absmax(X, None) == np.float32(9.0)
    assert O.act_tensor_absmax(np.zeros((2, 3), np.float32), None) == 0.0


def test_static_range_clips_runtime_outliers():
    """[P2] "Where it fits": the static level clips when a real input exceeds the
    calibrated range.  Inside the range the round trip is within half a step;
    beyond it the code is +-127 with the value's sign; a zero range gives codes 0
    and scale 1 (maitreyasuin page, zero-range case)."""
    rng = np.random.default_rng(23)
    s = rng.uniform(0.5, 2, 256).astype(np.float32)
    Xc = rng.standard_normal((64, 256)).astype(np.float32)
    clip = O.act_tensor_absmax(Xc, s)
    X = rng.standard_normal((64, 256)).astype(np.float32)
    X[5, 10] = 4 * clip * s[10]
    X[9, 11] = -6 * clip * s[11]
    Xq, xs = O.quant_act_static(X, s, clip)
    sc = np.float32(clip / np.float32(127))
    assert np.all(xs == sc)
    Xh = (X / s).astype(np.float32)
    inside = np.abs(Xh) <= clip
    assert not inside.all()
    err = np.abs(Xq.astype(np.float64) * sc - Xh)
    assert np.all(err[inside] <= 0.5 * sc * (1 + 1e-6))
    assert np.all(Xq[~inside] == np.sign(Xh[~inside]) * 127)
    assert Xq[5, 10] == 127 and Xq[9, 11] == -127
    assert int(Xq.min()) >= -127 and int(Xq.max()) <= 127
    q0, s0 = O.quant_act_static(X, s, 0.0)
    assert np.all(s0 == 1.0) and not q0.any()


# ------------------------------------ normalisation with the smoothing folded in
def _norm_case(seed, T=24, K=320):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, rng.choice(K, 4, replace=False)] *= 30
    X += np.float32(0.3) * rng.standard_normal((T, 1)).astype(np.float32)   # row offsets
    g = (1 + 0.2 * rng.standard_normal(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(K)).astype(np.float32)
    return X, g, b


@pytest.mark.parametrize("eps", [1e-6, 1e-2, 4.0])
def test_norms_match_library_float64(eps):
    """The textbook RMSNorm and LayerNorm (torch.nn.functional, float64) against
    the oracle's binary32 chain: every element within its few roundings."""
    import torch
    X, g, b = _norm_case(31)
    x64 = torch.from_numpy(X.astype(np.float64))
    K = X.shape[1]
    ref = torch.nn.functional.rms_norm(x64, (K,), torch.from_numpy(g.astype(np.float64)), eps).numpy()
    mean, rstd = O.norm_stats(X, "rms", eps)
    assert np.all(mean == 0)
    H = O.norm_apply(X, "rms", mean, rstd, g)
    assert np.all(np.abs(H - ref) <= 1e-6 * np.abs(ref) + 1e-30)
    ref = torch.nn.functional.layer_norm(x64, (K,), torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps).numpy()
    mean, rstd = O.norm_stats(X, "layer", eps)
    H = O.norm_apply(X, "layer", mean, rstd, g, b)
    tol = 1e-6 * (np.abs(ref) + np.abs(g)[None, :] * (np.abs(mean) * rstd)[:, None] + np.abs(b)[None, :])
    assert np.all(np.abs(H - ref) <= tol)


def test_norm_fold_equals_unfused_pipeline():
    """[P2] "Why the rescaling is free at runtime": normalising with gain g / s
    gives the same smoothed activations as normalising with g and then dividing
    by s, up to one rounding; the codes agree except for rare neighbours."""
    X, g, b = _norm_case(32, T=64, K=512)
    rng = np.random.default_rng(33)
    s = rng.uniform(0.2, 6.0, X.shape[1]).astype(np.float32)
    for kind, bias in (("rms", None), ("layer", b)):
        gf = O.fold_gain(g, s)
        bf = None if bias is None else O.fold_gain(bias, s)
        Xq, xs, mean, rstd = O.norm_quant_act(X, kind, gf, bf, eps=1e-6)
        H = O.norm_apply(X, kind, mean, rstd, g, bias)     # unfused: norm, then divide
        Xq2, xs2 = O.quant_act(H, s)
        np.testing.assert_allclose(xs, xs2, rtol=1e-6)
        d = np.abs(Xq.astype(int) - Xq2.astype(int))
        assert d.max() <= 1 and (d > 0).mean() < 1e-3, kind


def test_norm_zero_and_constant_rows():
    """A zero row normalises to zero (codes 0, scale 1, rstd = 1/sqrt(eps)); a
    constant row has zero variance, so LayerNorm returns the bias itself."""
    K = 64
    X = np.zeros((3, K), np.float32)
    X[1] = 2.5
    X[2] = np.linspace(-1, 1, K, dtype=np.float32)
    g = np.full(K, 1.5, np.float32)
    b = np.linspace(-3, 1, K, dtype=np.float32)
    Xq, xs, mean, rstd = O.norm_quant_act(X, "rms", g, eps=0.25)
    assert rstd[0] == 2.0 and xs[0] == 1.0 and not Xq[0].any()
    mean, rstd = O.norm_stats(X, "layer", 0.25)
    assert mean[1] == 2.5 and rstd[1] == 2.0
    H = O.norm_apply(X, "layer", mean, rstd, g, b)
    assert np.array_equal(H[1], b)
    Xq, xs, _, _ = O.norm_quant_act(X, "layer", g, b, eps=0.25)
    qb, sb = O.quant_act(b[None, :], None)
    assert np.array_equal(Xq[1], qb[0]) and xs[1] == sb[0]


def test_rms_scale_invariance():
    """With eps = 0, scaling a token by 4 scales mean(x^2) by 16 and rstd by 1/4
    exactly, so the codes and scales are unchanged."""
    X, g, _ = _norm_case(34)
    a = O.norm_quant_act(X, "rms", g, eps=0.0)
    c = O.norm_quant_act(X * np.float32(4), "rms", g, eps=0.0)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    assert np.array_equal(c[3] * np.float32(4), a[3])


def test_fold_gain_is_division():
    rng = np.random.default_rng(35)
    g = rng.uniform(-2, 2, 1000).astype(np.float32)
    s = rng.uniform(0.01, 50, 1000).astype(np.float32)
    assert np.array_equal(O.fold_gain(g, s), (g / s).astype(np.float32))


# ------------------------------------------- mixed-precision decomposition (P4, P5)
def _planted(seed, T=512, K=256, N=128, dims=(7, 23, 88, 154, 201), mult=14.0):
    """The structure of the maitreyasuin page's synthetic tensor (section "Route
    it, or move it"): standard-normal activations with a few input dimensions
    multiplied in every token, weights N(0, 0.1^2); drawn from our own stream."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, list(dims)] *= np.float32(mult)
    W = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    return X, W, np.array(sorted(dims), np.int32)


def test_decomp_select_ranks_by_max_magnitude():
    """maitreyasuin page: ranking dimensions by max magnitude recovers the planted
    ones; ties go to the lower index; the result is in ascending order."""
    X, _, dims = _planted(41)
    idx = O.decomp_select(O.col_absmax(X), 5)
    assert idx.tolist() == dims.tolist()
    a = np.array([1, 5, 3, 5, 5, 0.5], np.float32)
    assert O.decomp_select(a, 2).tolist() == [1, 3]
    assert O.decomp_select(a, 4).tolist() == [1, 2, 3, 4]
    assert O.decomp_select(a, 0).size == 0


def test_decomp_split_is_exact():
    """mercemay.com page, "Decomposition": the two products add up to the product
    of the concatenated operands (float64)."""
    X, W, dims = _planted(42, T=64)
    Xb, Xo = O.decomp_split(X, dims)
    Wb, Wo = O.decomp_split(W, dims)
    keep = np.setdiff1d(np.arange(X.shape[1]), dims)
    assert np.array_equal(Xb, X[:, keep]) and np.array_equal(Xo, X[:, dims])
    y = Xb.astype(np.float64) @ Wb.astype(np.float64).T + Xo.astype(np.float64) @ Wo.astype(np.float64).T
    Y = O.exact_product(X, W)
    assert np.linalg.norm(y - Y) <= 1e-12 * np.linalg.norm(Y)


def test_decomp_without_outliers_is_plain_w8a8():
    X, W, _ = _planted(43, T=40)
    none = np.zeros(0, np.int32)
    Wq, ws, Wo = O.decomp_prepare(W, none)
    y, Xq, xs, Xo, acc = O.decomp_linear(X, none, Wq, ws, Wo)
    y2, Xq2, xs2, acc2 = O.w8a8_linear(X, None, *O.quantize_weights(W, None))
    assert np.array_equal(y, y2) and np.array_equal(Xq, Xq2) and np.array_equal(acc, acc2)


def test_decomp_all_outliers_is_float_product():
    """Every channel kept in full precision: the layer is the binary32 product,
    within the recursive-summation bound K * 2^-24 * sum |x w| of the exact one."""
    X, W, _ = _planted(44, T=30, K=64, N=20, dims=(1, 2))
    idx = np.arange(64, dtype=np.int32)
    Wq, ws, Wo = O.decomp_prepare(W, idx)
    assert Wq.shape == (20, 0)
    y, *_ = O.decomp_linear(X, idx, Wq, ws, Wo)
    Y = O.exact_product(X, W)
    bound = 64 * 2.0 ** -24 * (np.abs(X).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert np.all(np.abs(y - Y) <= bound)
    assert np.abs(y - Y).max() > 0     # it is a binary32 sum, not the exact one


def test_decomp_bulk_scale_ignores_outliers():
    X = np.zeros((2, 16), np.float32)
    X[0, 3] = 1000.0      # outlier channel
    X[0, 5] = 1.27
    X[1, 3] = -2.0
    idx = np.array([3], np.int32)
    Xb, Xo = O.decomp_split(X, idx)
    Xq, xs = O.quant_act(Xb, None)
    assert xs[0] == np.float32(np.float32(1.27) / np.float32(127)) and xs[1] == 1.0
    assert Xo[:, 0].tolist() == [1000.0, -2.0]


def test_decomp_beats_one_grid():
    """[P5] "Route it, or move it" (105.4x on its own draw) and [P4]: keeping the
    planted dimensions in full precision cuts the W8A8 error by a large factor."""
    X, W, dims = _planted(45)
    plain = O.w8a8_relative_error(X, W, None)
    split = O.decomp_relative_error(X, W, O.decomp_select(O.col_absmax(X), 5))
    assert split * 4 < plain


# ------------------------------------------------------------------ FP8 E4M3 variant
def _torch_e4m3(v):
    import torch
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_library():
    import torch
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(O.e4m3_decode(codes), want)
    assert O.e4m3_decode(np.array([0x7E, 0x08, 0x01], np.uint8)).tolist() == [448.0, 2.0 ** -6, 2.0 ** -9]


def test_e4m3_encode_matches_library():
    """Nearest E4M3 value, ties to even, against torch's float8_e4m3fn cast on
    every grid point, every midpoint (ties), the binary32 neighbours of each
    midpoint and random values over the whole range (both signs)."""
    grid = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rng = np.random.default_rng(51)
    rnd = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(np.log(1e-4), np.log(448), 20000))])
    v = np.concatenate([grid, mids, near, rnd.astype(np.float32)])
    v = v[v <= 448].astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(O.e4m3_encode(v), _torch_e4m3(v))
    # saturation instead of NaN past the largest finite value
    assert O.e4m3_encode(np.array([448.0, 463.9, 1e6, -5e3], np.float32)).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_fp8_quantiser_rules():
    """scale = amax / 448, the row maximum maps to +-448 (code 0x7E / 0xFE), a
    zero row gets scale 1 and codes 0, and decoding times the scale is within
    half an E4M3 step (2^-4 relative for normal values) of the input."""
    rng = np.random.default_rng(52)
    X = (rng.standard_normal((6, 500)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32)
    X[3] = 0
    Xq, xs = O.quant_act_fp8(X, None)
    assert xs[3] == 1.0 and not Xq[3].any()
    for t in (0, 1, 2, 4, 5):
        amax = np.abs(X[t]).max()
        assert xs[t] == np.float32(amax / np.float32(448))
        k = int(np.argmax(np.abs(X[t])))
        assert Xq[t, k] == (0xFE if X[t, k] < 0 else 0x7E)
        d = O.e4m3_decode(Xq[t]).astype(np.float64) * xs[t]
        normal = np.abs(X[t]) >= 2.0 ** -6 * xs[t]
        assert np.all(np.abs(d - X[t])[normal] <= 2.0 ** -4 * np.abs(X[t])[normal])
        assert np.all(np.abs(d - X[t])[~normal] <= 2.0 ** -10 * xs[t] * 1.0001)


def test_page3_fp8(page3):
    """inferenceinterviews.com page, formats paragraph: FP8 3.3% before, 2.9%
    after smoothing on the same data."""
    X, W, _ = page3
    g = {r[0]: float(r[1]) for r in read_golden("page3_fp8.txt")}
    assert round(100 * O.fp8_relative_error(X, W, None), 1) == g["error_before_percent"]
    assert round(100 * O.fp8_relative_error(X, W, 0.5), 1) == g["error_after_alpha_0.5_percent"]


def test_fp8_dot_is_exact():
    """The binary64 sum of decoded E4M3 products equals integer arithmetic on the
    codes scaled by 2^18 (every product is a multiple of 2^-18)."""
    rng = np.random.default_rng(53)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    Xq = rng.choice(codes, (5, 300)).astype(np.uint8)
    Wq = rng.choice(codes, (7, 300)).astype(np.uint8)
    ti, ni = np.repeat(np.arange(5), 7), np.tile(np.arange(7), 5)
    acc, sab = O.fp8_dot_at(Xq, Wq, ti, ni)
    xi = (O.e4m3_decode(Xq).astype(np.float64) * 2 ** 9).astype(np.int64)
    wi = (O.e4m3_decode(Wq).astype(np.float64) * 2 ** 9).astype(np.int64)
    exact = (xi[ti] * wi[ni]).sum(1)
    assert np.array_equal(acc * 2.0 ** 18, exact.astype(np.float64))
    assert np.array_equal(sab * 2.0 ** 18, np.abs(xi[ti] * wi[ni]).sum(1).astype(np.float64))


def test_fp8_dot_full_matches_brute_force():
    """The full-matrix form (binary64 library product) equals the per-pair loop
    and pure-Python integer arithmetic on the codes, over the whole code range
    (subnormals, both signs, 448), with K long enough to cross row blocks."""
    rng = np.random.default_rng(59)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    Xq = rng.choice(codes, (9, 1100)).astype(np.uint8)
    Wq = rng.choice(codes, (6, 1100)).astype(np.uint8)
    Xq[0, :] = 0x7E                      # 448 everywhere: the largest products
    Wq[0, :] = 0x7E
    acc, sab = O.fp8_dot(Xq, Wq, rows=4)
    ti, ni = np.repeat(np.arange(9), 6), np.tile(np.arange(6), 9)
    acc_p, sab_p = O.fp8_dot_at(Xq, Wq, ti, ni)
    assert np.array_equal(acc[ti, ni], acc_p) and np.array_equal(sab[ti, ni], sab_p)
    dec = {c: O.e4m3_decode(np.array([c], np.uint8))[0] for c in range(256)}
    for t, n in ((0, 0), (3, 5), (8, 2)):
        # each decoded value times 2^9 is an integer, so this is exact
        ints = [int(dec[int(a)] * 512) * int(dec[int(b)] * 512) for a, b in zip(Xq[t], Wq[n])]
        assert acc[t, n] * 2.0 ** 18 == float(sum(ints))
        assert sab[t, n] * 2.0 ** 18 == float(sum(abs(v) for v in ints))
