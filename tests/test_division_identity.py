"""Host check of the arithmetic identity the quantiser kernels use for both of
the method's divisions (x / s_k and x_hat / scale):

    RN32(a / b) == RN32(RN64(a * r))     for binary32 a, b and r ~ 1/b in binary64

with r either the correctly rounded binary64 reciprocal or one a few ulps off (the
kernels form r from a hardware estimate refined by two Newton steps).  The proof
is that a/b never lies on a binary32 rounding midpoint and keeps a relative
distance of at least 2^-49 from every midpoint, while the binary64 route is off
by less than 2^-50.  This runs the same IEEE operations on the CPU.
"""
import numpy as np


def _check(a, b, ulps=0):
    a = a.astype(np.float32)
    b = b.astype(np.float32)
    want = a / b                                   # numpy float32 division: correctly rounded
    r = 1.0 / b.astype(np.float64)
    if ulps:
        r = r + ulps * np.spacing(r)
    got = (a.astype(np.float64) * r).astype(np.float32)
    bad = np.flatnonzero(want.view(np.uint32) != got.view(np.uint32))
    assert bad.size == 0, (a[bad[:5]], b[bad[:5]])


def test_random_pairs():
    rng = np.random.default_rng(0)
    for _ in range(20):
        a = rng.standard_normal(2_000_000).astype(np.float32) * np.exp(rng.uniform(-30, 30, 2_000_000))
        b = np.exp(rng.uniform(-20, 20, 2_000_000)).astype(np.float32)
        _check(a, b)
        _check(a, b, ulps=2)
        _check(a, b, ulps=-2)


def test_all_bf16_activations_against_many_factors():
    # every finite, normal bf16 value divided by 600 random factors
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (((np.abs(x) > 1e-30) & (np.abs(x) < 1e30)) | (x == 0))]
    rng = np.random.default_rng(1)
    for s in np.exp(rng.uniform(-8, 8, 600)).astype(np.float32):
        _check(x, np.full_like(x, s))


def test_quotients_next_to_midpoints():
    # b with all-ones significands and a chosen so that a/b falls close to a midpoint
    rng = np.random.default_rng(2)
    b = (np.float32(2.0) - np.spacing(np.float32(2.0)) * rng.integers(1, 64, 100000)).astype(np.float32)
    m = rng.integers(1 << 23, 1 << 24, 100000).astype(np.float64) + 0.5   # midpoints of [2^23, 2^24)
    a = (m * b.astype(np.float64)).astype(np.float32)
    _check(a, b)
    _check(np.nextafter(a, np.float32(np.inf)), b, ulps=1)
    _check(np.nextafter(a, np.float32(-np.inf)), b, ulps=-1)


def test_scale_quotients_of_the_quantiser():
    # x_hat / (amax / 127) for values up to amax: the second division
    rng = np.random.default_rng(3)
    for _ in range(10):
        amax = np.float32(np.exp(rng.uniform(-10, 10)))
        scale = np.float32(amax / np.float32(127.0))
        x = (rng.uniform(-1, 1, 3_000_000) * amax).astype(np.float32)
        _check(x, np.full_like(x, scale))
        _check(x, np.full_like(x, scale), ulps=1)
