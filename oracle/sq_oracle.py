"""NumPy front end of the plain C oracle (sq_oracle.c) -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the benchmark's CPU-baseline leg use this module;
the product path must never import it.  It shares no code with the HIP library.

Each function cites the passage it follows (pages by title, section named):
  [P2] multigrid.ai "SmoothQuant Explained"
  [P3] inferenceinterviews.com "Why do activation outliers break INT8 W8A8..."
  [P4] mercemay.com "Activation Outlier Channels and Mixed-Precision Decomposition"
  [P5] maitreyasuin.github.io "...01-one-outlier"

bf16 inputs are widened to float32 exactly before they reach the C code; the
diagnostics (exact product, relative error, channel ratios) are float64.

Parity pins of every function live in tests/test_oracle_pins.py; none of the
functions here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsqoracle.so")
_lib = None
_lock = threading.Lock()

__all__ = ["build", "col_absmax", "smooth_scales", "quantize_weights", "quant_act",
           "int_gemm", "int_gemm_at", "dequant", "dequant_at", "to_bf16", "w8a8_linear",
           "prepare", "w8a8_relative_error", "channel_max_over_median", "exact_product",
           "widen_bf16", "set_threads", "act_tensor_absmax", "quant_act_static",
           "quant_act_per_tensor", "fold_gain", "norm_stats", "norm_apply", "norm_quant_act",
           "decomp_select", "decomp_split", "decomp_outlier_product", "decomp_prepare",
           "decomp_linear", "decomp_relative_error", "e4m3_encode", "e4m3_decode",
           "quantize_weights_fp8", "quant_act_fp8", "fp8_dot_at", "fp8_dot", "fp8_relative_error"]

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall"]


def build(force: bool = False) -> str:
    """Compile sq_oracle.c with gcc into oracle/libsqoracle.so."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            F = ctypes.c_float
            lib.sqo_col_absmax.argtypes = [P, I64, I64, P]
            lib.sqo_smooth_scales.argtypes = [P, P, I64, F, P]
            lib.sqo_quantize_weights.argtypes = [P, I64, I64, P, P, P]
            lib.sqo_quant_act.argtypes = [P, I64, I64, P, P, P]
            lib.sqo_int_gemm.argtypes = [P, P, I64, I64, I64, P]
            lib.sqo_int_gemm.restype = ctypes.c_int
            lib.sqo_int_gemm_at.argtypes = [P, P, I64, P, P, I64, P]
            lib.sqo_int_gemm_at.restype = ctypes.c_int
            lib.sqo_dequant.argtypes = [P, P, P, I64, I64, P]
            lib.sqo_dequant_at.argtypes = [P, P, P, P, P, I64, P]
            lib.sqo_to_bf16.argtypes = [P, I64, P]
            lib.sqo_act_tensor_absmax.argtypes = [P, I64, I64, P]
            lib.sqo_act_tensor_absmax.restype = F
            lib.sqo_quant_act_static.argtypes = [P, I64, I64, P, F, P, P]
            lib.sqo_quant_act_static.restype = None
            lib.sqo_fold_gain.argtypes = [P, P, I64, P]
            lib.sqo_norm_stats.argtypes = [P, I64, I64, ctypes.c_int, F, P, P]
            lib.sqo_norm_apply.argtypes = [P, I64, I64, ctypes.c_int, P, P, P, P, P]
            for f in ("sqo_fold_gain", "sqo_norm_stats", "sqo_norm_apply"):
                getattr(lib, f).restype = None
            lib.sqo_decomp_select.argtypes = [P, I64, I64, P]
            lib.sqo_decomp_split.argtypes = [P, I64, I64, P, I64, P, P]
            lib.sqo_decomp_outlier_product.argtypes = [P, P, I64, I64, I64, P]
            lib.sqo_add.argtypes = [P, P, I64, P]
            for f in ("sqo_decomp_select", "sqo_decomp_split", "sqo_decomp_outlier_product", "sqo_add"):
                getattr(lib, f).restype = None
            lib.sqo_e4m3_encode.argtypes = [F]
            lib.sqo_e4m3_encode.restype = ctypes.c_uint8
            lib.sqo_e4m3_decode.argtypes = [ctypes.c_uint8]
            lib.sqo_e4m3_decode.restype = F
            lib.sqo_quantize_weights_fp8.argtypes = [P, I64, I64, P, P, P]
            lib.sqo_quant_act_fp8.argtypes = [P, I64, I64, P, P, P]
            lib.sqo_fp8_dot_at.argtypes = [P, P, I64, P, P, I64, P, P]
            for f in ("sqo_quantize_weights_fp8", "sqo_quant_act_fp8", "sqo_fp8_dot_at"):
                getattr(lib, f).restype = None
            for f in ("sqo_col_absmax", "sqo_smooth_scales", "sqo_quantize_weights",
                      "sqo_quant_act", "sqo_dequant", "sqo_dequant_at", "sqo_to_bf16"):
                getattr(lib, f).restype = None
            _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """OpenMP thread count for the oracle (the CPU baseline reports it)."""
    os.environ["OMP_NUM_THREADS"] = str(n)
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(ctypes.c_int(n))
    except OSError:
        pass


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32, exactly (the bits become the high half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def col_absmax(A: np.ndarray) -> np.ndarray:
    """[P3] max_t |X_tj| (activations) or max_n |W_nj| (weights), per column j."""
    A = _f32(A)
    out = np.empty(A.shape[1], np.float32)
    _load().sqo_col_absmax(_ptr(A), A.shape[0], A.shape[1], _ptr(out))
    return out


def smooth_scales(x_absmax, w_absmax, alpha: float) -> np.ndarray:
    """[P2] section "Alpha: how much difficulty to move"; [P3] "A strong answer";
    [P5] "Route it, or move it" (maxima clamped at 1e-8):
    s_j = max(xa_j, 1e-8)^alpha / max(wa_j, 1e-8)^(1 - alpha), binary64 then
    rounded to binary32."""
    xa, wa = _f32(x_absmax), _f32(w_absmax)
    assert xa.shape == wa.shape
    s = np.empty_like(xa)
    _load().sqo_smooth_scales(_ptr(xa), _ptr(wa), xa.size, float(alpha), _ptr(s))
    return s


def quantize_weights(W, s=None):
    """[P3] W_hat = W diag(s); per-output-channel symmetric int8 ([P5] "The four
    operations").  Returns (Wq int8 [N,K], w_scale float32 [N])."""
    W = _f32(W)
    N, K = W.shape
    s = None if s is None else _f32(s)
    Wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    _load().sqo_quantize_weights(_ptr(W), N, K, _ptr(s), _ptr(Wq), _ptr(ws))
    return Wq, ws


def quant_act(X, s=None):
    """[P3] X_hat = X diag(s)^-1; dynamic per-token symmetric int8 ([P5] "The
    four operations").  Returns (Xq int8 [T,K], x_scale float32 [T])."""
    X = _f32(X)
    T, K = X.shape
    s = None if s is None else _f32(s)
    Xq = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    _load().sqo_quant_act(_ptr(X), T, K, _ptr(s), _ptr(Xq), _ptr(xs))
    return Xq, xs


def act_tensor_absmax(X, s=None) -> np.float32:
    """[P2] section "Where it fits, and where it does not" (O2 / O3: one
    activation scale per tensor); [P1] "Activations are a distribution": the
    range of the smoothed tensor, max over all t, k of |X_tk / s_k|."""
    X = _f32(X)
    T, K = X.shape
    s = None if s is None else _f32(s)
    return np.float32(_load().sqo_act_tensor_absmax(_ptr(X), T, K, _ptr(s)))


def quant_act_static(X, s, clip):
    """[P5] "The four operations" with a given range (quantize_dequantize's
    clip): scale = clip / 127, codes clamp(round(X_tk / s_k / scale)), values past
    the range clamp to +-127; clip = 0 gives codes 0 and scale 1.  Returns
    (Xq int8 [T,K], x_scale float32 [T], every entry the tensor's scale)."""
    X = _f32(X)
    T, K = X.shape
    s = None if s is None else _f32(s)
    clip = np.float32(clip)
    assert np.isfinite(clip) and clip >= 0
    Xq = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    _load().sqo_quant_act_static(_ptr(X), T, K, _ptr(s), float(clip), _ptr(Xq), _ptr(xs))
    return Xq, xs


def quant_act_per_tensor(X, s=None):
    """Dynamic per-tensor activation quantisation (O2): the static quantiser with
    the tensor's own range.  Returns (Xq, x_scale [T], amax)."""
    amax = act_tensor_absmax(X, s)
    Xq, xs = quant_act_static(X, s, amax)
    return Xq, xs, amax


NORM_KINDS = {"rms": 0, "layer": 1}


def fold_gain(v, s):
    """[P2] "Why the rescaling is free at runtime"; [P3] "A strong answer": fold
    diag(s)^-1 into the preceding norm's gain (or bias): v / s per channel."""
    v, s = _f32(v), _f32(s)
    assert v.shape == s.shape and v.ndim == 1
    out = np.empty_like(v)
    _load().sqo_fold_gain(_ptr(v), _ptr(s), v.size, _ptr(out))
    return out


def norm_stats(X, kind, eps):
    """Per-token (mean, rstd) of the textbook RMSNorm / LayerNorm (binary64 sums,
    rounded once); mean is 0 for RMSNorm."""
    X = _f32(X)
    T, K = X.shape
    mean = np.empty(T, np.float32)
    rstd = np.empty(T, np.float32)
    _load().sqo_norm_stats(_ptr(X), T, K, NORM_KINDS[kind], float(np.float32(eps)), _ptr(mean),
                           _ptr(rstd))
    return mean, rstd


def norm_apply(X, kind, mean, rstd, gain, bias=None):
    """h = ((x - mean) * rstd) * gain (+ bias), binary32, one rounding per op."""
    X = _f32(X)
    T, K = X.shape
    mean, rstd, gain = _f32(mean), _f32(rstd), _f32(gain)
    assert mean.size == T and rstd.size == T and gain.size == K
    bias = None if bias is None else _f32(bias)
    H = np.empty((T, K), np.float32)
    _load().sqo_norm_apply(_ptr(X), T, K, NORM_KINDS[kind], _ptr(mean), _ptr(rstd), _ptr(gain),
                           _ptr(bias), _ptr(H))
    return H


def norm_quant_act(X, kind, gain, bias=None, eps=1e-6, stats=None):
    """The producer in front of the layer: normalisation with the smoothing
    folded into its gain (and bias), then dynamic per-token int8 of the result.
    `stats` = (mean, rstd) replaces the oracle's own statistics (to compare codes
    given the same binary32 statistics).  Returns (Xq, x_scale, mean, rstd)."""
    mean, rstd = norm_stats(X, kind, eps) if stats is None else (_f32(stats[0]), _f32(stats[1]))
    H = norm_apply(X, kind, mean, rstd, gain, bias)
    Xq, xs = quant_act(H, None)
    return Xq, xs, mean, rstd


def decomp_select(absmax, n_o):
    """[P4] "Decomposition" (a static outlier set chosen from calibration); [P5]
    (dimensions ranked by max magnitude): the n_o input channels with the largest
    absolute maximum, ties to the lower index, returned in ascending order."""
    a = _f32(absmax)
    assert 0 <= n_o <= a.size
    idx = np.empty(n_o, np.int32)
    _load().sqo_decomp_select(_ptr(a), a.size, int(n_o), _ptr(idx))
    return idx


def decomp_split(A, idx):
    """(A[:, keep], A[:, idx]) with keep the complement of idx, both in order."""
    A = _f32(A)
    rows, K = A.shape
    idx = np.ascontiguousarray(idx, np.int32)
    assert np.all(np.diff(idx) > 0) and (idx.size == 0 or (idx[0] >= 0 and idx[-1] < K))
    bulk = np.empty((rows, K - idx.size), np.float32)
    outl = np.empty((rows, idx.size), np.float32)
    _load().sqo_decomp_split(_ptr(A), rows, K, _ptr(idx), idx.size, _ptr(bulk), _ptr(outl))
    return bulk, outl


def decomp_outlier_product(Xo, Wo):
    """[P4] y_out = x_out @ W_out.T in binary32 (sum over the outlier channels in
    ascending order, one rounding per operation)."""
    Xo, Wo = _f32(Xo), _f32(Wo)
    T, n_o = Xo.shape
    N, n_o2 = Wo.shape
    assert n_o == n_o2
    Yo = np.empty((T, N), np.float32)
    _load().sqo_decomp_outlier_product(_ptr(Xo), _ptr(Wo), T, N, n_o, _ptr(Yo))
    return Yo


def decomp_prepare(W, idx):
    """Offline half: bulk weight columns quantised per output channel; outlier
    columns kept in binary32.  Returns (Wq_bulk, w_scale, W_out)."""
    Wb, Wo = decomp_split(W, idx)
    Wq, ws = quantize_weights(Wb, None)
    return Wq, ws, Wo


def decomp_linear(X, idx, Wq_bulk, w_scale, W_out):
    """Runtime half ([P4] split_outlier_matmul; [P5] split reduction): bulk
    activation columns quantised per token, integer matmul with the float
    epilogue, plus the binary32 product of the outlier columns, added once.
    Returns (y float32 [T,N], Xq_bulk, x_scale, X_out, acc)."""
    Xb, Xo = decomp_split(X, idx)
    Xq, xs = quant_act(Xb, None)
    acc = int_gemm(Xq, Wq_bulk)
    yb = dequant(acc, xs, w_scale)
    yo = decomp_outlier_product(Xo, W_out)
    y = np.empty_like(yb)
    _load().sqo_add(_ptr(yb), _ptr(yo), yb.size, _ptr(y))
    return y, Xq, xs, Xo, acc


def decomp_relative_error(X, W, idx):
    """||Y_decomp - Y|| / ||Y|| against the exact float64 product."""
    Wq, ws, Wo = decomp_prepare(W, idx)
    y, *_ = decomp_linear(X, idx, Wq, ws, Wo)
    Y = exact_product(X, W)
    return float(np.linalg.norm(y.astype(np.float64) - Y) / np.linalg.norm(Y))


def e4m3_encode(v):
    """[P3] formats paragraph, FP8 E4M3: nearest E4M3 code (ties to the even
    code), saturated at +-448; elementwise over an array."""
    v = np.asarray(v, np.float32)
    lib = _load()
    out = np.array([lib.sqo_e4m3_encode(float(x)) for x in v.ravel()], np.uint8)
    return out.reshape(v.shape)


def e4m3_decode(c):
    """E4M3 code -> binary32 value (exact)."""
    c = np.asarray(c, np.uint8)
    lib = _load()
    lut = np.array([lib.sqo_e4m3_decode(i) for i in range(256)], np.float32)
    return lut[c]


def quantize_weights_fp8(W, s=None):
    """FP8 E4M3 per-output-channel codes of W diag(s): scale = row amax / 448.
    Returns (Wq uint8 [N,K] E4M3 codes, w_scale float32 [N])."""
    W = _f32(W)
    N, K = W.shape
    s = None if s is None else _f32(s)
    Wq = np.empty((N, K), np.uint8)
    ws = np.empty(N, np.float32)
    _load().sqo_quantize_weights_fp8(_ptr(W), N, K, _ptr(s), _ptr(Wq), _ptr(ws))
    return Wq, ws


def quant_act_fp8(X, s=None):
    """FP8 E4M3 per-token codes of X diag(s)^-1.  Returns (Xq uint8, x_scale)."""
    X = _f32(X)
    T, K = X.shape
    s = None if s is None else _f32(s)
    Xq = np.empty((T, K), np.uint8)
    xs = np.empty(T, np.float32)
    _load().sqo_quant_act_fp8(_ptr(X), T, K, _ptr(s), _ptr(Xq), _ptr(xs))
    return Xq, xs


def fp8_dot_at(Xq, Wq, ti, ni):
    """Exact (binary64) dot products of decoded codes at (t, n) pairs, and the
    sums of |products|."""
    Xq = np.ascontiguousarray(Xq, np.uint8)
    Wq = np.ascontiguousarray(Wq, np.uint8)
    ti = np.ascontiguousarray(ti, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    assert Xq.shape[1] == Wq.shape[1] and ti.shape == ni.shape
    acc = np.empty(ti.size, np.float64)
    sab = np.empty(ti.size, np.float64)
    _load().sqo_fp8_dot_at(_ptr(Xq), _ptr(Wq), Xq.shape[1], _ptr(ti), _ptr(ni), ti.size, _ptr(acc),
                           _ptr(sab))
    return acc, sab


def fp8_dot(Xq, Wq, rows=2048):
    """Exact dot products of decoded E4M3 codes for every (t, n), and the sums of
    |products| ([P3] formats paragraph: the FP8 layer's accumulator is the sum of
    the code products).  Computed as binary64 matrix products of the decoded
    codes, `rows` tokens at a time.  That is exact in any summation order: every
    E4M3 value is a multiple of 2^-9 with |v| <= 448, so every product is a
    multiple of 2^-18 below 2^18 in magnitude, and for K <= 2^16 every partial
    sum is a multiple of 2^-18 below 2^34, which binary64 holds exactly; the
    library product therefore gives the same values as fp8_dot_at's loop."""
    Xq = np.ascontiguousarray(Xq, np.uint8)
    Wq = np.ascontiguousarray(Wq, np.uint8)
    assert Xq.shape[1] == Wq.shape[1] and Xq.shape[1] <= 1 << 16
    lut = e4m3_decode(np.arange(256)).astype(np.float64)
    wv = lut[Wq].T.copy()
    wa = np.abs(wv)
    T, N = Xq.shape[0], Wq.shape[0]
    acc = np.empty((T, N), np.float64)
    sab = np.empty((T, N), np.float64)
    for t0 in range(0, T, rows):
        xv = lut[Xq[t0:t0 + rows]]
        acc[t0:t0 + rows] = xv @ wv
        sab[t0:t0 + rows] = np.abs(xv) @ wa
    return acc, sab


def fp8_relative_error(X, W, alpha):
    """[P3]: relative Frobenius error of the layer with FP8 E4M3 per-token
    activations and per-output-channel weights (exact accumulation, binary32
    epilogue); alpha=None: no smoothing."""
    X32, W32 = _f32(X), _f32(W)
    if alpha is None:
        s = None
    else:
        s = smooth_scales(col_absmax(X32), col_absmax(W32), alpha)
    Wq, ws = quantize_weights_fp8(W32, s)
    Xq, xs = quant_act_fp8(X32, s)
    lut = e4m3_decode(np.arange(256)).astype(np.float64)
    acc = lut[Xq] @ lut[Wq].T
    y = (acc.astype(np.float32) * (xs[:, None] * ws[None, :])).astype(np.float64)
    Y = exact_product(X, W)
    return float(np.linalg.norm(y - Y) / np.linalg.norm(Y))


def int_gemm(Xq, Wq):
    """[P5] "Which scales factor out": acc_tn = sum_k P_tk Q_nk, exact int32."""
    Xq = np.ascontiguousarray(Xq, np.int8)
    Wq = np.ascontiguousarray(Wq, np.int8)
    T, K = Xq.shape
    N, K2 = Wq.shape
    assert K == K2
    acc = np.empty((T, N), np.int32)
    if _load().sqo_int_gemm(_ptr(Xq), _ptr(Wq), T, N, K, _ptr(acc)):
        raise OverflowError("integer accumulator does not fit int32")
    return acc


def int_gemm_at(Xq, Wq, ti, ni):
    """acc at the listed (t, n) pairs only."""
    Xq = np.ascontiguousarray(Xq, np.int8)
    Wq = np.ascontiguousarray(Wq, np.int8)
    ti = np.ascontiguousarray(ti, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    assert ti.shape == ni.shape and Xq.shape[1] == Wq.shape[1]
    assert ti.size == 0 or (ti.min() >= 0 and ti.max() < Xq.shape[0])
    assert ni.size == 0 or (ni.min() >= 0 and ni.max() < Wq.shape[0])
    acc = np.empty(ti.size, np.int32)
    if _load().sqo_int_gemm_at(_ptr(Xq), _ptr(Wq), Xq.shape[1], _ptr(ti), _ptr(ni),
                               ti.size, _ptr(acc)):
        raise OverflowError("integer accumulator does not fit int32")
    return acc


def dequant(acc, x_scale, w_scale):
    """[P4] section "Decomposition": (qx @ qW.T) * (sx * sw) --
    y = fl32(fl32(acc) * fl32(xs_t * ws_n))."""
    acc = np.ascontiguousarray(acc, np.int32)
    xs, ws = _f32(x_scale), _f32(w_scale)
    T, N = acc.shape
    assert xs.size == T and ws.size == N
    y = np.empty((T, N), np.float32)
    _load().sqo_dequant(_ptr(acc), _ptr(xs), _ptr(ws), T, N, _ptr(y))
    return y


def dequant_at(acc, x_scale, w_scale, ti, ni):
    acc = np.ascontiguousarray(acc, np.int32)
    xs, ws = _f32(x_scale), _f32(w_scale)
    ti = np.ascontiguousarray(ti, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    y = np.empty(acc.size, np.float32)
    _load().sqo_dequant_at(_ptr(acc), _ptr(xs), _ptr(ws), _ptr(ti), _ptr(ni), acc.size, _ptr(y))
    return y


def to_bf16(y) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), nearest, ties to even."""
    y = _f32(y)
    out = np.empty(y.shape, np.uint16)
    _load().sqo_to_bf16(_ptr(y), y.size, _ptr(out))
    return out


def prepare(X_stats, W, alpha):
    """Offline half of the layer: statistics, smoothing factors, smoothed and
    quantised weights.  alpha=None means no smoothing (s is None)."""
    if alpha is None:
        Wq, ws = quantize_weights(W, None)
        return dict(s=None, x_absmax=None, w_absmax=None, Wq=Wq, w_scale=ws)
    xa = col_absmax(X_stats)
    wa = col_absmax(W)
    s = smooth_scales(xa, wa, alpha)
    Wq, ws = quantize_weights(W, s)
    return dict(s=s, x_absmax=xa, w_absmax=wa, Wq=Wq, w_scale=ws)


def w8a8_linear(X, s, Wq, w_scale, act="token"):
    """Runtime half: quantisation of X diag(s)^-1 (act="token": one scale per
    token; act="tensor": one scale for the tensor, dynamic), integer GEMM,
    epilogue.  Returns (y float32 [T,N], Xq, x_scale, acc)."""
    if act == "token":
        Xq, xs = quant_act(X, s)
    elif act == "tensor":
        Xq, xs, _ = quant_act_per_tensor(X, s)
    else:
        raise ValueError(act)
    acc = int_gemm(Xq, Wq)
    return dequant(acc, xs, w_scale), Xq, xs, acc


def exact_product(X, W):
    """Y = X W^T in float64 ([P5]: Y = X W^T, X in R^{T x K}, W in R^{N x K})."""
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64).T


def w8a8_relative_error(X, W, alpha, act="token"):
    """[P3] relative Frobenius error ||Y_q - Y|| / ||Y|| of the W8A8 layer with
    per-token (act="token") or per-tensor (act="tensor") activation scales and
    per-output-channel weights; alpha=None: no smoothing.  Statistics are taken
    from X itself, as in [P3]'s experiment."""
    X32, W32 = _f32(X), _f32(W)
    p = prepare(X32, W32, alpha)
    y, *_ = w8a8_linear(X32, p["s"], p["Wq"], p["w_scale"], act=act)
    Y = exact_product(X, W)
    return float(np.linalg.norm(y.astype(np.float64) - Y) / np.linalg.norm(Y))


def channel_max_over_median(A):
    """[P3] table "alpha / act max/median / weight max/median": the largest
    per-input-channel max divided by the median per-input-channel max (median of
    an even count is the mean of the two middle values)."""
    m = col_absmax(A).astype(np.float64)
    return float(m.max() / np.median(m))
