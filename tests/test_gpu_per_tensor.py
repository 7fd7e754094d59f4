"""Parity of the per-tensor activation path (sq_act_absmax, sq_quant_act_static,
sq_quant_act_per_tensor) with the CPU oracle, through the C ABI.

Bar: the tensor range, the scale and every int8 code bit-exact (the oracle is fed
the same smoothing factors); GEMM outputs as for the per-token path.
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


def _acts(rng, T, K, dtype, n_out=3, mult=40.0):
    X = rng.standard_normal((T, K)).astype(np.float32)
    if K > n_out:
        X[:, rng.choice(K, n_out, replace=False)] *= np.float32(mult)
    if dtype == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    return X


def _s(rng, K):
    return rng.uniform(0.3, 4.0, K).astype(np.float32)


SHAPES = [(1, 1), (37, 80), (37, 83), (300, 1000), (1025, 8), (5000, 24), (64, 16384), (5, 20000)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K", SHAPES)
@pytest.mark.parametrize("smooth", [False, True])
def test_act_absmax(sq, dtype, T, K, smooth):
    rng = np.random.default_rng(T * 31 + K)
    X = _acts(rng, T, K, dtype)
    s = _s(rng, K) if smooth else None
    sd = torch.from_numpy(s).to(DEV) if smooth else None
    Xd = dev_act(X, dtype)
    want = O.act_tensor_absmax(X, s)
    got = host(sq.sq_act_absmax(Xd, sd))
    assert got[0] == want
    # running maximum: a larger previous value survives, a smaller one is replaced
    big = torch.tensor([float(want) * 3 + 1], device=DEV)
    assert host(sq.sq_act_absmax(Xd, sd, amax=big, accumulate=True))[0] == np.float32(float(want) * 3 + 1)
    small = torch.tensor([float(want) / 2], device=DEV)
    assert host(sq.sq_act_absmax(Xd, sd, amax=small, accumulate=True))[0] == want
    # scalar kernels (misaligned rows) give the same value
    if T * K > 1:
        assert host(sq.sq_act_absmax(misaligned(Xd), sd))[0] == want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K", SHAPES)
def test_quant_act_static_calibrated_range(sq, dtype, T, K):
    """Range from a separate calibration draw: runtime values beyond it clamp."""
    rng = np.random.default_rng(T * 17 + K + 5)
    s = _s(rng, K)
    Xc = _acts(rng, max(T // 2, 1), K, dtype)
    X = _acts(rng, T, K, dtype)
    X[0, 0] = X[0, 0] * 8 + np.float32(3.0)     # exceeds the calibrated range
    if dtype == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).float().numpy()
    clip = O.act_tensor_absmax(Xc, s)
    sd = torch.from_numpy(s).to(DEV)
    clip_d = torch.tensor([float(clip)], dtype=torch.float32, device=DEV)
    Xd = dev_act(X, dtype)
    Xq, xs = sq.sq_quant_act_static(Xd, sd, clip_d)
    Xq_r, xs_r = O.quant_act_static(X, s, clip)
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)
    assert int(Xq_r.min()) >= -127
    if T * K > 1:
        Xq2, xs2 = sq.sq_quant_act_static(misaligned(Xd), sd, clip_d)
        assert np.array_equal(host(Xq2), Xq_r) and np.array_equal(host(xs2), xs_r)


def test_quant_act_static_edges(sq):
    """The 127.6-step edge (clip 127 gives scale 1), a zero range (codes 0,
    scale 1), and no smoothing vector."""
    row = np.array([127.6, -127.6, 128.4, 500.0, -1e4, 126.5, 0.5, -0.5, 1.5, 2.5, -2.5, 0.0,
                    3.5, 4.5, -126.5, 126.49], np.float32)
    X = np.tile(row, (3, 2))
    Xd = dev_act(X, "f32")
    for clip in (127.0, 0.0, 1e4, 3.0):
        clip_d = torch.tensor([clip], dtype=torch.float32, device=DEV)
        Xq, xs = sq.sq_quant_act_static(Xd, None, clip_d)
        Xq_r, xs_r = O.quant_act_static(X, None, clip)
        assert np.array_equal(host(Xq), Xq_r), clip
        assert np.array_equal(host(xs), xs_r), clip
    Xq, xs = sq.sq_quant_act_static(Xd, None, torch.tensor([127.0], device=DEV))
    assert host(Xq)[0, :5].tolist() == [127, -127, 127, 127, -127]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K", [(1, 1), (37, 83), (300, 1000), (64, 16384), (5, 20000), (2048, 4096)])
def test_quant_act_per_tensor(sq, dtype, T, K):
    rng = np.random.default_rng(T + 7 * K)
    X = _acts(rng, T, K, dtype)
    X[T // 2] = 0.0
    s = _s(rng, K)
    sd = torch.from_numpy(s).to(DEV)
    Xq, xs, amax = sq.sq_quant_act_per_tensor(dev_act(X, dtype), sd)
    Xq_r, xs_r, amax_r = O.quant_act_per_tensor(X, s)
    assert host(amax)[0] == amax_r
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)


def test_per_tensor_zero_tensor(sq):
    Xd = torch.zeros((33, 64), device=DEV)
    Xq, xs, amax = sq.sq_quant_act_per_tensor(Xd, None)
    assert host(amax)[0] == 0.0 and np.all(host(xs) == 1.0) and not host(Xq).any()


def test_per_tensor_linear_tiny_page(sq):
    """Per-tensor codes through the GEMM: exact accumulators, fp32 outputs equal
    to the oracle's layer with per-tensor activations."""
    for name in ("tiny_t128_k1024_n1024", "page_t512_k4096_n4096"):
        w = WL.make(name)
        p = O.prepare(w.X, w.W, 0.5)
        s = torch.from_numpy(p["s"]).to(DEV)
        Wq = torch.from_numpy(p["Wq"]).to(DEV)
        ws = torch.from_numpy(p["w_scale"]).to(DEV)
        Xq, xs, _ = sq.sq_quant_act_per_tensor(dev_act(w.X, w.x_dtype), s)
        y = sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.float32)
        acc = sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=torch.int32)
        y_r, Xq_r, xs_r, acc_r = O.w8a8_linear(w.X, p["s"], p["Wq"], p["w_scale"], act="tensor")
        assert np.array_equal(host(Xq), Xq_r) and np.array_equal(host(xs), xs_r)
        assert np.array_equal(host(acc), acc_r)
        assert_out_close(host(y), y_r, "f32")


def test_per_tensor_full_size_heavy(sq):
    """Heavy-outlier prefill activations X bf16 [8192 x 8192] with the smoothing
    factors of the benchmark's configuration: range, scales and all codes; then
    the static quantiser with a calibration range taken on the first 512 tokens
    (which later tokens exceed)."""
    w = WL.make("heavy_t8192_k8192_n8192")
    xa, wa = O.col_absmax(w.X), O.col_absmax(w.W)
    s = O.smooth_scales(xa, wa, w.alpha)
    sd = torch.from_numpy(s).to(DEV)
    Xd = dev_act(w.X, w.x_dtype)
    Xq, xs, amax = sq.sq_quant_act_per_tensor(Xd, sd)
    Xq_r, xs_r, amax_r = O.quant_act_per_tensor(w.X, s)
    assert host(amax)[0] == amax_r
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)
    calib = sq.sq_act_absmax(Xd[:512], sd)
    clip_r = O.act_tensor_absmax(w.X[:512], s)
    assert host(calib)[0] == clip_r
    Xq, xs = sq.sq_quant_act_static(Xd, sd, calib)
    Xq_r, xs_r = O.quant_act_static(w.X, s, clip_r)
    assert np.array_equal(host(xs), xs_r)
    assert np.array_equal(host(Xq), Xq_r)
    assert clip_r < amax_r and (np.abs(Xq_r) == 127).sum() > 0
