"""Parity of the fused normalisation + per-token int8 producer (sq_norm_quant_act)
and of the gain fold (sq_fold_norm_gain) with the CPU oracle, through the C ABI.

Bar: folded gains bit-exact; the per-token statistics (rounded once to binary32)
within 1e-6 relative of the oracle's binary64 ones (the mean within 1e-6 of |mean| plus
one standard deviation); codes and scales bit-exact once the oracle is given the
same binary32 statistics, and equal to the oracle's own codes except where its
statistics round differently.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, dev_act, host, misaligned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _case(seed, T, K, dtype):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)).astype(np.float32)
    if K > 4:
        X[:, rng.choice(K, 3, replace=False)] *= 25
    X += np.float32(0.5) * rng.standard_normal((T, 1)).astype(np.float32)
    if dtype == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    g = (1 + 0.2 * rng.standard_normal(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(K)).astype(np.float32)
    s = rng.uniform(0.2, 5.0, K).astype(np.float32)
    return X, g, b, s


def _check(sq, X, dtype, kind, g, b, eps, Xd=None):
    gd = torch.from_numpy(g).to(DEV)
    bd = None if b is None else torch.from_numpy(b).to(DEV)
    Xd = dev_act(X, dtype) if Xd is None else Xd
    Xq, xs, mean, rstd = sq.sq_norm_quant_act(Xd, kind, gd, bd, eps=eps)
    Xq, xs, mean, rstd = host(Xq), host(xs), host(mean), host(rstd)
    mean_r, rstd_r = O.norm_stats(X, kind, eps)
    np.testing.assert_allclose(rstd, rstd_r, rtol=1e-6, atol=0)
    assert np.all(np.abs(mean - mean_r) <= 1e-6 * (np.abs(mean_r) + 1.0 / rstd_r))
    Xq_r, xs_r, _, _ = O.norm_quant_act(X, kind, g, b, eps=eps, stats=(mean, rstd))
    assert np.array_equal(xs, xs_r)
    assert np.array_equal(Xq, Xq_r)
    # against the oracle's own statistics: identical wherever they round alike
    same = (mean == mean_r) & (rstd == rstd_r)
    Xq_o, xs_o, _, _ = O.norm_quant_act(X, kind, g, b, eps=eps)
    assert np.array_equal(Xq[same], Xq_o[same]) and np.array_equal(xs[same], xs_o[same])
    # The kernel sums each 8-element chunk of squares in binary32 with fused
    # multiply-adds (chunk sums in binary64): for non-negative terms the mean
    # square is then within 8 * 2^-24 relative of the binary64 one (LayerNorm:
    # 10 * 2^-24, its centred differences being rounded once more), so rstd is
    # within half of that before its final rounding, and the two rounded values
    # differ by at most that plus one binary32 ulp.  Rows whose binary64 value
    # lies that close to a rounding boundary round apart; with few chunks per row
    # (short K) that can be most rows, so no share of equal rows is asserted.
    delta = (5.0 if kind == "layer" else 4.0) * 2.0 ** -24
    r64 = rstd_r.astype(np.float64)
    ulp = np.spacing(np.abs(rstd_r)).astype(np.float64)
    assert np.all(np.abs(rstd.astype(np.float64) - r64) <= delta * r64 + ulp)
    return Xq, xs


# (800, 2056) and (1537, 2048): more rows than workgroups (3 per CU), so each
# workgroup walks several rows and its last prefetch re-reads row R - 1
SHAPES = [(1, 8), (37, 80), (37, 83), (300, 1000), (64, 4096), (33, 16384), (5, 20000), (800, 2056), (1537, 2048)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K", SHAPES)
@pytest.mark.parametrize("kind,with_bias", [("rms", False), ("layer", False), ("layer", True)])
def test_norm_quant(sq, dtype, T, K, kind, with_bias):
    X, g, b, s = _case(T * 13 + K, T, K, dtype)
    gf, bf = O.fold_gain(g, s), (O.fold_gain(b, s) if with_bias else None)
    _check(sq, X, dtype, kind, gf, bf, 1e-6)
    if T * K > 8:
        _check(sq, X, dtype, kind, gf, bf, 1e-6, Xd=misaligned(dev_act(X, dtype)))


def test_fold_norm_gain(sq):
    rng = np.random.default_rng(3)
    for K in (1, 255, 8192, 10001):
        g = rng.uniform(-2, 2, K).astype(np.float32)
        s = rng.uniform(0.01, 40, K).astype(np.float32)
        out = sq.sq_fold_norm_gain(torch.from_numpy(g).to(DEV), torch.from_numpy(s).to(DEV))
        assert np.array_equal(host(out), O.fold_gain(g, s))


def test_norm_zero_constant_rows_and_eps(sq):
    K = 256
    X = np.zeros((4, K), np.float32)
    X[1] = 2.5
    X[2] = np.linspace(-1, 1, K, dtype=np.float32)
    X[3] = 1e-3
    g = np.full(K, 1.5, np.float32)
    b = np.linspace(-3, 1, K, dtype=np.float32)
    for eps in (0.25, 1e-6, 0.0):
        Xq, xs = _check(sq, X[1:] if eps == 0.0 else X, "f32", "rms", g, None, eps)
        if eps > 0:
            assert xs[0] == 1.0 and not Xq[0].any()
    Xq, xs = _check(sq, X, "f32", "layer", g, b, 0.25)
    qb, sb = O.quant_act(b[None, :], None)
    assert np.array_equal(Xq[1], qb[0]) and xs[1] == sb[0]


@pytest.mark.parametrize("name", ["prefill_t2048_k4096_n16384", "heavy_t8192_k8192_n8192"])
def test_norm_quant_full_size(sq, name):
    """The workload's activations taken as the norm's input (RMSNorm, gain
    ~1 +- 0.2 folded with smoothing factors from the normalised activations):
    all statistics, scales and codes at full size."""
    w = WL.make(name)
    rng = np.random.default_rng(77)
    K = w.K
    g = (1 + 0.2 * rng.standard_normal(K)).astype(np.float32)
    mean, rstd = O.norm_stats(w.X[:512], "rms", 1e-6)
    H = O.norm_apply(w.X[:512], "rms", mean, rstd, g)
    s = O.smooth_scales(O.col_absmax(H), O.col_absmax(w.W), w.alpha)
    gf = O.fold_gain(g, s)
    gfd = sq.sq_fold_norm_gain(torch.from_numpy(g).to(DEV), torch.from_numpy(s).to(DEV))
    assert np.array_equal(host(gfd), gf)
    _check(sq, w.X, w.x_dtype, "rms", gf, None, 1e-6)
