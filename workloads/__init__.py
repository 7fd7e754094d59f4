"""Seeded synthetic inputs for the SmoothQuant W8A8 linear layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no smoothing, no quantization, no products).  Both the CPU
oracle's tests and the HIP path's tests and benchmark take their inputs from
here, so that the two sides see the same bytes.

The recipe follows the synthetic experiments on the pages:
  * inferenceinterviews.com, "Why do activation outliers break INT8 W8A8...",
    section "A strong answer" (its NumPy experiment): standard-normal
    activations, a few outlier channels multiplied into every token, weights
    standard-normal times 0.02;
  * maitreyasuin.github.io, "...01-one-outlier", section "Where transformer
    activations put their outliers": the same outlier dimensions in every token.

Five workloads are named after what they are (token count x input width x
output width); each has a fixed seed.  bf16 activations are produced by
rounding the fp32 draw to bfloat16 with torch's own conversion (round to
nearest even), so every bf16 value is also held exactly as an fp32 array.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make", "make_linear", "bf16_bits", "from_bf16_bits",
           "page3_experiment_data", "page_tiny_fixture"]


@dataclasses.dataclass
class Workload:
    """One linear-layer problem instance.

    X       float32 [T, K]  activations (bf16-representable when x_dtype == "bf16")
    W       float32 [N, K]  weights, row n = output channel n, K contiguous
    X_calib float32 [Tc, K] or None: separate calibration draw (same outlier
            channels and multipliers, fresh noise); None means the smoothing
            statistics come from X itself
    alpha   migration strength(s)
    x_dtype "f32" or "bf16"; y_dtype "f32" or "bf16"
    outliers  int64 [n_out] outlier channel indices; mult float32 [n_out]
    """
    name: str
    X: np.ndarray
    W: np.ndarray
    X_calib: Optional[np.ndarray]
    alphas: tuple
    x_dtype: str
    y_dtype: str
    outliers: np.ndarray
    mult: np.ndarray
    seed: int

    @property
    def T(self):
        return self.X.shape[0]

    @property
    def K(self):
        return self.X.shape[1]

    @property
    def N(self):
        return self.W.shape[0]

    @property
    def alpha(self):
        return self.alphas[0]

    @property
    def stats_source(self):
        """Activations the smoothing statistics are taken from."""
        return self.X if self.X_calib is None else self.X_calib


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32 (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float32 array -> uint16 bit patterns (exact truncation)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_outliers(rng, K, n_out, mult_range):
    idx = np.sort(rng.choice(K, n_out, replace=False)).astype(np.int64)
    lo, hi = mult_range
    if lo == hi:
        mult = np.full(n_out, lo, dtype=np.float32)
    else:  # log-uniform on [lo, hi]
        mult = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n_out)).astype(np.float32)
    return idx, mult


def _acts(rng, T, K, dtype):
    return rng.standard_normal((T, K), dtype=dtype)


def _plant(X, idx, mult):
    if len(idx):
        X[:, idx] *= mult[None, :]
    return X


def make_linear(T, N, K, *, n_out=0, mult_range=(60.0, 60.0), seed=0, x_dtype="f32",
                y_dtype="f32", alphas=(0.5,), calib_tokens=None, w_std=0.02,
                name=None, draw_dtype=np.float32, channels_after_acts=False) -> Workload:
    """Generic seeded outlier-structured linear problem (any shape).

    Order of draws from numpy's PCG64 stream seeded with `seed`: outlier channel
    indices, multipliers, activations [T, K], weights [N, K]; with
    channels_after_acts the activations come first.  The calibration draw, when
    asked for, uses its own stream seeded with seed + 100.  draw_dtype float64
    keeps the draw (and X, W) in float64 instead of float32; such a draw is
    used as float64 data (x_dtype must stay "f32").
    """
    rng = np.random.default_rng(seed)
    if channels_after_acts:
        X = _acts(rng, T, K, draw_dtype)
        idx, mult = _draw_outliers(rng, K, n_out, mult_range)
    else:
        idx, mult = _draw_outliers(rng, K, n_out, mult_range)
        X = _acts(rng, T, K, draw_dtype)
    X = _plant(X, idx, mult)
    W = rng.standard_normal((N, K), dtype=draw_dtype)
    W *= W.dtype.type(w_std)
    Xc = None
    if calib_tokens:
        Xc = _plant(_acts(np.random.default_rng(seed + 100), calib_tokens, K, draw_dtype), idx, mult)
    if x_dtype == "bf16" and draw_dtype == np.float32:
        X = _round_bf16(X)
        if Xc is not None:
            Xc = _round_bf16(Xc)
    elif x_dtype != "f32":
        raise ValueError(x_dtype)
    return Workload(name or f"linear_T{T}_N{N}_K{K}", X, W, Xc, tuple(alphas), x_dtype,
                    y_dtype, idx, mult, seed)


# name -> (T, N, K, n_outliers, multiplier range, x dtype, y dtype, alphas, calibration tokens)
WORKLOADS = {
    # tiny linear: 4 fixed outlier channels x60 in every token
    "tiny_t128_k1024_n1024": dict(T=128, N=1024, K=1024, n_out=4, mult_range=(60., 60.),
                                  x_dtype="f32", y_dtype="f32", alphas=(0.5,), calib_tokens=None),
    # page-style: 6 outlier channels x60, three migration strengths
    "page_t512_k4096_n4096": dict(T=512, N=4096, K=4096, n_out=6, mult_range=(60., 60.),
                                  x_dtype="f32", y_dtype="f32", alphas=(0.0, 0.5, 1.0),
                                  calib_tokens=None),
    # decode-shaped skinny GEMM: 16 tokens, 0.5% outlier channels x20..x80 log-uniform
    "decode_t16_k8192_n28672": dict(T=16, N=28672, K=8192, n_out=41, mult_range=(20., 80.),
                                    x_dtype="bf16", y_dtype="bf16", alphas=(0.5,),
                                    calib_tokens=512),
    # prefill FFN up-projection of a 6.7B-class model: 0.2% outliers x30..x100
    "prefill_t2048_k4096_n16384": dict(T=2048, N=16384, K=4096, n_out=8, mult_range=(30., 100.),
                                       x_dtype="bf16", y_dtype="bf16", alphas=(0.5,),
                                       calib_tokens=512),
    # heavy-outlier large prefill: 30% outlier channels x10..x60
    "heavy_t8192_k8192_n8192": dict(T=8192, N=8192, K=8192, n_out=2458, mult_range=(10., 60.),
                                    x_dtype="bf16", y_dtype="bf16", alphas=(0.75,),
                                    calib_tokens=None),
}
_SEEDS = {name: 1001 + i for i, name in enumerate(WORKLOADS)}


def make(name: str, *, tokens: Optional[int] = None) -> Workload:
    """Build a named workload.  `tokens` truncates T (the first rows of the same
    draw are kept, so a sample is a prefix of the full problem)."""
    cfg = dict(WORKLOADS[name])
    w = make_linear(seed=_SEEDS[name], name=name, **cfg)
    if tokens is not None and tokens < w.T:
        w.X = np.ascontiguousarray(w.X[:tokens])
    return w


def page3_experiment_data():
    """The synthetic data of the NumPy experiment on inferenceinterviews.com,
    "Why do activation outliers break INT8 W8A8..." (section "A strong answer"):
    seed 0; 512 tokens x 4096 channels, standard normal; 6 distinct channels
    multiplied by 60 in every token; 1024 output channels, standard normal
    weights times 0.02.  The printed figures depend on the exact stream, so the
    draw is made in float64 with the channels chosen after the activations, in
    the experiment's order.  Returns (X, W, outlier channels), float64."""
    w = make_linear(512, 1024, 4096, n_out=6, mult_range=(60.0, 60.0), seed=0,
                    draw_dtype=np.float64, channels_after_acts=True, name="page3_experiment")
    return w.X, w.W, w.outliers


def page_tiny_fixture(seed=7, T=37, N=45, K=80):
    """Small ragged problem for tests (T, N, K deliberately not tile multiples)."""
    return make_linear(T, N, K, n_out=3, mult_range=(20., 60.), seed=seed)
