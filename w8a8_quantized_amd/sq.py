"""Python binding of libsq.so (include/sq.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are torch
tensors on the current HIP device (PyTorch provides the device memory and the
stream; all arithmetic runs in the library's kernels).  Outputs that are not
passed in are allocated with torch.empty.  A non-OK status raises RuntimeError
with the library's status string.  There is no fallback: if libsq.so is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsq.so")

SQ_F32, SQ_BF16, SQ_I32 = 0, 1, 2
SQ_NORM_RMS, SQ_NORM_LAYER = 0, 1
_NORM = {"rms": SQ_NORM_RMS, "layer": SQ_NORM_LAYER}
SQ_MAX_K = 133144
SQ_NOALLOC_SCRATCH_BYTES = 32 << 20
_DT = {torch.float32: SQ_F32, torch.bfloat16: SQ_BF16, torch.int32: SQ_I32}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m w8a8_quantized_amd.build` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _F, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "sq_status_string": ([_I], ctypes.c_char_p),
    "sq_col_absmax": ([_P, _I, _I64, _I64, _P, _I, _P], _I),
    "sq_smooth_scales_from_absmax": ([_P, _P, _I64, _F, _P, _P], _I),
    "sq_smooth_scales": ([_P, _I, _I64, _P, _I, _I64, _I64, _F, _P, _P, _P, _P], _I),
    "sq_quantize_weights": ([_P, _I, _I64, _I64, _P, _P, _P, _P], _I),
    "sq_quant_act": ([_P, _I, _I64, _I64, _P, _P, _P, _P], _I),
    "sq_act_absmax": ([_P, _I, _I64, _I64, _P, _P, _I, _P], _I),
    "sq_quant_act_static": ([_P, _I, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "sq_quant_act_per_tensor": ([_P, _I, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "sq_fold_norm_gain": ([_P, _P, _I64, _P, _P], _I),
    "sq_norm_quant_act": ([_P, _I, _I64, _I64, _I, _P, _P, _F, _P, _P, _P, _P, _P], _I),
    "sq_decomp_select": ([_P, _I64, _I64, _P, _P, _P], _I),
    "sq_decomp_prepare_weights": ([_P, _I, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P], _I),
    "sq_decomp_quant_act": ([_P, _I, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P], _I),
    "sq_decomp_gemm": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _P], _I),
    "sq_quantize_weights_fp8": ([_P, _I, _I64, _I64, _P, _P, _P, _P], _I),
    "sq_quant_act_fp8": ([_P, _I, _I64, _I64, _P, _P, _P, _P], _I),
    "sq_fp8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "sq_w8a8_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "sq_w8a8_linear_workspace_size": ([_I64, _I64], _SZ),
    "sq_w8a8_linear": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P], _I),
    "sq_w8a8_linear_noalloc": ([_P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


def sq_status_string(status: int) -> str:
    return _lib.sq_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(sq_status_string(rc))


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t, allowed=(torch.float32, torch.bfloat16)):
    if t.dtype not in allowed:
        raise ValueError(f"dtype {t.dtype} not accepted (expected one of {allowed})")
    return _DT[t.dtype]


def _vec(t, n, name, dev, dtype=torch.float32, optional=False):
    """Check a per-channel / per-token vector argument: n entries of `dtype` on
    the device `dev` (None accepted when optional).  A short or wrongly typed
    vector would be read past its end by the kernels, so it is refused here."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.numel() != n or t.dtype != dtype or t.device != torch.device(dev):
        raise ValueError(f"{name} must be a {dtype} tensor of {n} entries on {dev} "
                         f"(got {t.dtype}, {t.numel()} entries on {t.device})")
    return t


def _want(t, shape, dtype, dev):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != torch.device(dev):
        raise ValueError(f"output must be {dtype} of shape {tuple(shape)} on {dev}")
    return t


def sq_col_absmax(A, amax=None, accumulate=False):
    """amax[j] = max_i |A[i, j]| (running max if accumulate)."""
    rows, cols = A.shape
    amax = _want(amax, (cols,), torch.float32, A.device)
    _check(_lib.sq_col_absmax(_ptr(A), _dt(A), rows, cols, _ptr(amax), int(bool(accumulate)),
                              _stream(A.device)))
    return amax


def sq_smooth_scales_from_absmax(x_absmax, w_absmax, alpha, s=None):
    """s = max(xa,1e-8)^alpha / max(wa,1e-8)^(1-alpha)."""
    K = x_absmax.numel()
    _vec(x_absmax, K, "x_absmax", x_absmax.device)
    _vec(w_absmax, K, "w_absmax", x_absmax.device)
    s = _want(s, (K,), torch.float32, x_absmax.device)
    _check(_lib.sq_smooth_scales_from_absmax(_ptr(x_absmax), _ptr(w_absmax), K, float(alpha),
                                             _ptr(s), _stream(x_absmax.device)))
    return s


def sq_smooth_scales(X, W, alpha, s=None, x_absmax=None, w_absmax=None, maxima=(True, True)):
    """Smoothing factors from a calibration batch X [T, K] and weights W [N, K].
    Returns (s, x_absmax, w_absmax).  maxima = (False, ...) / (..., False)
    passes NULL for that column-maxima output (the library then keeps no copy;
    it is returned as None)."""
    T, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("X and W differ in K")
    dev = X.device
    if W.device != dev:
        raise ValueError("X and W must be on the same device")
    s = _want(s, (K,), torch.float32, dev)
    x_absmax = _want(x_absmax, (K,), torch.float32, dev) if maxima[0] else None
    w_absmax = _want(w_absmax, (K,), torch.float32, dev) if maxima[1] else None
    _check(_lib.sq_smooth_scales(_ptr(X), _dt(X), T, _ptr(W), _dt(W), N, K, float(alpha), _ptr(s),
                                 _ptr(x_absmax), _ptr(w_absmax), _stream(dev)))
    return s, x_absmax, w_absmax


def sq_quantize_weights(W, s=None, Wq=None, w_scale=None):
    """Per-output-channel int8 weights of W diag(s).  Returns (Wq, w_scale)."""
    N, K = W.shape
    _vec(s, K, "s", W.device, optional=True)
    Wq = _want(Wq, (N, K), torch.int8, W.device)
    w_scale = _want(w_scale, (N,), torch.float32, W.device)
    _check(_lib.sq_quantize_weights(_ptr(W), _dt(W), N, K, _ptr(s), _ptr(Wq), _ptr(w_scale),
                                    _stream(W.device)))
    return Wq, w_scale


def sq_quant_act(X, s=None, Xq=None, x_scale=None):
    """Dynamic per-token int8 codes of X diag(s)^-1.  Returns (Xq, x_scale)."""
    T, K = X.shape
    _vec(s, K, "s", X.device, optional=True)
    Xq = _want(Xq, (T, K), torch.int8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    _check(_lib.sq_quant_act(_ptr(X), _dt(X), T, K, _ptr(s), _ptr(Xq), _ptr(x_scale),
                             _stream(X.device)))
    return Xq, x_scale


def sq_act_absmax(X, s=None, amax=None, accumulate=False):
    """Range of X diag(s)^-1 over the whole tensor, as a device float [1]."""
    T, K = X.shape
    _vec(s, K, "s", X.device, optional=True)
    amax = _want(amax, (1,), torch.float32, X.device)
    _check(_lib.sq_act_absmax(_ptr(X), _dt(X), T, K, _ptr(s), _ptr(amax), int(bool(accumulate)),
                              _stream(X.device)))
    return amax


def sq_quant_act_static(X, s, clip, Xq=None, x_scale=None):
    """Per-tensor int8 codes of X diag(s)^-1 against the range clip (device float
    [1]).  Returns (Xq, x_scale), every x_scale entry the tensor's scale."""
    T, K = X.shape
    _vec(s, K, "s", X.device, optional=True)
    _vec(clip, 1, "clip", X.device)
    Xq = _want(Xq, (T, K), torch.int8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    _check(_lib.sq_quant_act_static(_ptr(X), _dt(X), T, K, _ptr(s), _ptr(clip), _ptr(Xq),
                                    _ptr(x_scale), _stream(X.device)))
    return Xq, x_scale


def sq_quant_act_per_tensor(X, s=None, amax=None, Xq=None, x_scale=None):
    """Dynamic per-tensor int8 codes of X diag(s)^-1.  Returns (Xq, x_scale, amax)."""
    T, K = X.shape
    _vec(s, K, "s", X.device, optional=True)
    amax = _want(amax, (1,), torch.float32, X.device)
    Xq = _want(Xq, (T, K), torch.int8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    _check(_lib.sq_quant_act_per_tensor(_ptr(X), _dt(X), T, K, _ptr(s), _ptr(amax), _ptr(Xq),
                                        _ptr(x_scale), _stream(X.device)))
    return Xq, x_scale, amax


def sq_fold_norm_gain(v, s, out=None):
    """v / s per channel (a norm's gain or bias with the smoothing folded in)."""
    _vec(s, v.numel(), "s", v.device)
    _vec(v, v.numel(), "v", v.device)
    out = _want(out, (v.numel(),), torch.float32, v.device)
    _check(_lib.sq_fold_norm_gain(_ptr(v), _ptr(s), v.numel(), _ptr(out), _stream(v.device)))
    return out


def sq_norm_quant_act(X, kind, gain, bias=None, eps=1e-6, Xq=None, x_scale=None, mean=None,
                      rstd=None):
    """RMSNorm / LayerNorm (kind "rms" / "layer") with folded gain, then per-token
    int8.  Returns (Xq, x_scale, mean, rstd)."""
    T, K = X.shape
    if kind not in _NORM:
        raise ValueError(f"kind must be one of {tuple(_NORM)}")
    _vec(gain, K, "gain", X.device)
    _vec(bias, K, "bias", X.device, optional=True)
    Xq = _want(Xq, (T, K), torch.int8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    mean = _want(mean, (T,), torch.float32, X.device)
    rstd = _want(rstd, (T,), torch.float32, X.device)
    _check(_lib.sq_norm_quant_act(_ptr(X), _dt(X), T, K, _NORM[kind], _ptr(gain), _ptr(bias),
                                  float(eps), _ptr(Xq), _ptr(x_scale), _ptr(mean), _ptr(rstd),
                                  _stream(X.device)))
    return Xq, x_scale, mean, rstd


def sq_decomp_select(absmax, n_o, idx=None, mask=None):
    """The n_o channels of largest absmax (ascending) and the 0/1 column mask."""
    K = absmax.numel()
    _vec(absmax, K, "absmax", absmax.device)
    idx = _want(idx, (n_o,), torch.int32, absmax.device)
    mask = _want(mask, (K,), torch.float32, absmax.device)
    _check(_lib.sq_decomp_select(_ptr(absmax), K, int(n_o), _ptr(idx) if n_o else None, _ptr(mask),
                                 _stream(absmax.device)))
    return idx, mask


def sq_decomp_prepare_weights(W, mask, idx, Wq=None, w_scale=None, W_out=None):
    """Bulk int8 weights (outlier columns zeroed), w_scale, W_out [n_o, N]."""
    N, K = W.shape
    n_o = idx.numel()
    _vec(mask, K, "mask", W.device)
    _vec(idx, n_o, "idx", W.device, dtype=torch.int32)
    Wq = _want(Wq, (N, K), torch.int8, W.device)
    w_scale = _want(w_scale, (N,), torch.float32, W.device)
    W_out = _want(W_out, (n_o, N), torch.float32, W.device)
    _check(_lib.sq_decomp_prepare_weights(_ptr(W), _dt(W), N, K, _ptr(mask), _ptr(idx) if n_o else None,
                                          n_o, _ptr(Wq), _ptr(w_scale), _ptr(W_out) if n_o else None,
                                          _stream(W.device)))
    return Wq, w_scale, W_out


def sq_decomp_quant_act(X, mask, idx, Xq=None, x_scale=None, X_out=None):
    """Bulk per-token int8 codes (outlier columns zeroed), x_scale, X_out [n_o, T]."""
    T, K = X.shape
    n_o = idx.numel()
    _vec(mask, K, "mask", X.device)
    _vec(idx, n_o, "idx", X.device, dtype=torch.int32)
    Xq = _want(Xq, (T, K), torch.int8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    X_out = _want(X_out, (n_o, T), torch.float32, X.device)
    _check(_lib.sq_decomp_quant_act(_ptr(X), _dt(X), T, K, _ptr(mask), _ptr(idx) if n_o else None, n_o,
                                    _ptr(Xq), _ptr(x_scale), _ptr(X_out) if n_o else None,
                                    _stream(X.device)))
    return Xq, x_scale, X_out


def sq_decomp_gemm(Xq, x_scale, Wq, w_scale, X_out, W_out, out_dtype=torch.bfloat16, Y=None):
    """dequant(Xq @ Wq^T) + X_out^T @ W_out (binary32), fused in one launch."""
    T, K = Xq.shape
    N, K2 = Wq.shape
    n_o = X_out.shape[0]
    if K != K2 or tuple(W_out.shape) != (n_o, N) or X_out.shape[1] != T:
        raise ValueError("shapes: Xq [T, K], Wq [N, K], X_out [n_o, T], W_out [n_o, N]")
    if Xq.dtype != torch.int8 or Wq.dtype != torch.int8 or Wq.device != Xq.device:
        raise ValueError("Xq and Wq must be int8 on the same device")
    _vec(x_scale, T, "x_scale", Xq.device)
    _vec(w_scale, N, "w_scale", Xq.device)
    _vec(X_out, n_o * T, "X_out", Xq.device)
    _vec(W_out, n_o * N, "W_out", Xq.device)
    yt = _DT.get(out_dtype)
    if yt is None or out_dtype == torch.int32:
        raise ValueError(f"out_dtype {out_dtype} not accepted")
    Y = _want(Y, (T, N), out_dtype, Xq.device)
    _check(_lib.sq_decomp_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale),
                               _ptr(X_out) if n_o else None, _ptr(W_out) if n_o else None, T, N, K, n_o,
                               _ptr(Y), yt, _stream(Xq.device)))
    return Y


def sq_quantize_weights_fp8(W, s=None, Wq=None, w_scale=None):
    """Per-output-channel FP8 E4M3 codes (uint8) of W diag(s).  Returns (Wq, w_scale)."""
    N, K = W.shape
    _vec(s, K, "s", W.device, optional=True)
    Wq = _want(Wq, (N, K), torch.uint8, W.device)
    w_scale = _want(w_scale, (N,), torch.float32, W.device)
    _check(_lib.sq_quantize_weights_fp8(_ptr(W), _dt(W), N, K, _ptr(s), _ptr(Wq), _ptr(w_scale),
                                        _stream(W.device)))
    return Wq, w_scale


def sq_quant_act_fp8(X, s=None, Xq=None, x_scale=None):
    """Per-token FP8 E4M3 codes (uint8) of X diag(s)^-1.  Returns (Xq, x_scale)."""
    T, K = X.shape
    _vec(s, K, "s", X.device, optional=True)
    Xq = _want(Xq, (T, K), torch.uint8, X.device)
    x_scale = _want(x_scale, (T,), torch.float32, X.device)
    _check(_lib.sq_quant_act_fp8(_ptr(X), _dt(X), T, K, _ptr(s), _ptr(Xq), _ptr(x_scale),
                                 _stream(X.device)))
    return Xq, x_scale


def sq_fp8_gemm(Xq, x_scale, Wq, w_scale, out_dtype=torch.bfloat16, Y=None):
    """Y = dequant(e4m3(Xq) @ e4m3(Wq)^T) on the FP8 matrix cores."""
    T, K = Xq.shape
    N, K2 = Wq.shape
    if K != K2 or Xq.dtype != torch.uint8 or Wq.dtype != torch.uint8 or Wq.device != Xq.device:
        raise ValueError("Xq [T, K] and Wq [N, K] must be uint8 E4M3 codes with the same K, on one device")
    _vec(x_scale, T, "x_scale", Xq.device)
    _vec(w_scale, N, "w_scale", Xq.device)
    yt = _DT.get(out_dtype)
    if yt is None or out_dtype == torch.int32:
        raise ValueError(f"out_dtype {out_dtype} not accepted")
    Y = _want(Y, (T, N), out_dtype, Xq.device)
    _check(_lib.sq_fp8_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), T, N, K, _ptr(Y), yt,
                            _stream(Xq.device)))
    return Y


def sq_w8a8_gemm(Xq, x_scale, Wq, w_scale, out_dtype=torch.bfloat16, Y=None):
    """Y = dequant(Xq @ Wq^T); out_dtype torch.int32 returns the raw accumulators."""
    T, K = Xq.shape
    N, K2 = Wq.shape
    if K != K2 or Xq.dtype != torch.int8 or Wq.dtype != torch.int8 or Wq.device != Xq.device:
        raise ValueError("Xq [T, K] and Wq [N, K] must be int8 with the same K, on one device")
    yt = _DT.get(out_dtype)
    if yt is None:
        raise ValueError(f"out_dtype {out_dtype} not accepted")
    # the raw int32 accumulators need no scales (they may be None)
    _vec(x_scale, T, "x_scale", Xq.device, optional=out_dtype == torch.int32)
    _vec(w_scale, N, "w_scale", Xq.device, optional=out_dtype == torch.int32)
    Y = _want(Y, (T, N), out_dtype, Xq.device)
    _check(_lib.sq_w8a8_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), T, N, K, _ptr(Y),
                             yt, _stream(Xq.device)))
    return Y


def sq_w8a8_linear_workspace_size(T, K):
    return int(_lib.sq_w8a8_linear_workspace_size(int(T), int(K)))


def sq_w8a8_linear(X, s, Wq, w_scale, out_dtype=torch.bfloat16, Y=None, workspace=None):
    """Run-time layer: per-token quantisation of X diag(s)^-1, then the W8A8 GEMM."""
    T, K = X.shape
    N, K2 = Wq.shape
    if K != K2 or Wq.dtype != torch.int8 or Wq.device != X.device:
        raise ValueError("Wq must be int8 [N, K] on X's device")
    _vec(s, K, "s", X.device, optional=True)
    _vec(w_scale, N, "w_scale", X.device)
    yt = _DT.get(out_dtype)
    if yt is None or out_dtype == torch.int32:
        raise ValueError(f"out_dtype {out_dtype} not accepted")
    Y = _want(Y, (T, N), out_dtype, X.device)
    need = sq_w8a8_linear_workspace_size(T, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check(_lib.sq_w8a8_linear(_ptr(X), _dt(X), _ptr(s), _ptr(Wq), _ptr(w_scale), T, N, K, _ptr(Y),
                               yt, _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(X.device)))
    return Y


def sq_w8a8_linear_noalloc(X, s, Wq, w_scale, Y, out_dtype=torch.bfloat16):
    """sq_w8a8_linear with the workspace in the library's fixed per-GPU scratch
    (for callers that cannot allocate): Y must be passed in; calls that overlap
    on one GPU race."""
    T, K = X.shape
    N, K2 = Wq.shape
    if K != K2 or Wq.dtype != torch.int8 or Wq.device != X.device:
        raise ValueError("Wq must be int8 [N, K] on X's device")
    _vec(s, K, "s", X.device, optional=True)
    _vec(w_scale, N, "w_scale", X.device)
    yt = _DT.get(out_dtype)
    if yt is None or out_dtype == torch.int32:
        raise ValueError(f"out_dtype {out_dtype} not accepted")
    if Y is None:
        raise ValueError("Y must be passed in (this call allocates nothing)")
    Y = _want(Y, (T, N), out_dtype, X.device)
    _check(_lib.sq_w8a8_linear_noalloc(_ptr(X), _dt(X), _ptr(s), _ptr(Wq), _ptr(w_scale), T, N, K, _ptr(Y),
                                       yt, _stream(X.device)))
    return Y
