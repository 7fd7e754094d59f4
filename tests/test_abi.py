"""C ABI checks that need no GPU: libsq.so loads, exports every entry point that
include/sq.h declares, and rejects bad arguments on the host before touching
the device (these calls return before any HIP runtime call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "w8a8_quantized_amd", "libsq.so")
HEADER = os.path.join(ROOT, "include", "sq.h")

(SQ_OK, SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALPHA, SQ_ERR_DTYPE, SQ_ERR_WORKSPACE, SQ_ERR_HIP,
 SQ_ERR_ARG, SQ_ERR_SCRATCH) = range(9)
F32, BF16, I32 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    L = ctypes.CDLL(LIB)
    P, I64, F, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    L.sq_status_string.restype = ctypes.c_char_p
    L.sq_status_string.argtypes = [I]
    L.sq_col_absmax.argtypes = [P, I, I64, I64, P, I, P]
    L.sq_smooth_scales_from_absmax.argtypes = [P, P, I64, F, P, P]
    L.sq_smooth_scales.argtypes = [P, I, I64, P, I, I64, I64, F, P, P, P, P]
    L.sq_quantize_weights.argtypes = [P, I, I64, I64, P, P, P, P]
    L.sq_quant_act.argtypes = [P, I, I64, I64, P, P, P, P]
    L.sq_w8a8_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
    L.sq_w8a8_linear_workspace_size.argtypes = [I64, I64]
    L.sq_w8a8_linear_workspace_size.restype = ctypes.c_size_t
    L.sq_w8a8_linear.argtypes = [P, I, P, P, P, I64, I64, I64, P, I, P, ctypes.c_size_t, P]
    L.sq_act_absmax.argtypes = [P, I, I64, I64, P, P, I, P]
    L.sq_quant_act_static.argtypes = [P, I, I64, I64, P, P, P, P, P]
    L.sq_quant_act_per_tensor.argtypes = [P, I, I64, I64, P, P, P, P, P]
    L.sq_fold_norm_gain.argtypes = [P, P, I64, P, P]
    L.sq_norm_quant_act.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P, P, P]
    return L


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for name in ("sq_smooth_scales", "sq_quantize_weights", "sq_quant_act", "sq_w8a8_gemm",
                 "sq_w8a8_linear"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_header():
    src = open(os.path.join(ROOT, "w8a8_quantized_amd", "sq.py")).read()
    for name in declared_functions():
        assert re.search(rf"^def {name}\(", src, flags=re.M), name


def test_status_strings(lib):
    for code in range(9):
        s = lib.sq_status_string(code).decode()
        assert s.startswith("SQ_"), s
    assert b"unknown" in lib.sq_status_string(99)


# A fake non-NULL device address: validation fails before any use of it.
FAKE = ctypes.c_void_p(0x1000)


def test_null_pointers_rejected(lib):
    assert lib.sq_col_absmax(None, F32, 4, 4, FAKE, 0, None) == SQ_ERR_NULL
    assert lib.sq_col_absmax(FAKE, F32, 4, 4, None, 0, None) == SQ_ERR_NULL
    assert lib.sq_quant_act(None, F32, 4, 4, None, FAKE, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_quant_act(FAKE, F32, 4, 4, None, None, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_quantize_weights(FAKE, F32, 4, 4, None, FAKE, None, None) == SQ_ERR_NULL
    assert lib.sq_smooth_scales(FAKE, F32, 4, FAKE, F32, 4, 4, 0.5, None, FAKE, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_smooth_scales(None, F32, 4, FAKE, F32, 4, 4, 0.5, FAKE, None, None, None) == SQ_ERR_NULL
    assert lib.sq_smooth_scales_from_absmax(FAKE, None, 4, 0.5, FAKE, None) == SQ_ERR_NULL
    # scales are required unless the output is the raw int32 accumulator
    assert lib.sq_w8a8_gemm(FAKE, None, FAKE, FAKE, 4, 4, 16, FAKE, F32, None) == SQ_ERR_NULL
    assert lib.sq_w8a8_gemm(FAKE, FAKE, None, FAKE, 4, 4, 16, FAKE, I32, None) == SQ_ERR_NULL
    assert lib.sq_w8a8_linear(FAKE, BF16, None, FAKE, None, 4, 4, 16, FAKE, BF16, FAKE, 1 << 20,
                              None) == SQ_ERR_NULL


def test_shapes_rejected(lib):
    for r, c in ((0, 4), (4, 0), (-1, 4)):
        assert lib.sq_col_absmax(FAKE, F32, r, c, FAKE, 0, None) == SQ_ERR_SHAPE
        assert lib.sq_quant_act(FAKE, F32, r, c, None, FAKE, FAKE, None) == SQ_ERR_SHAPE
        assert lib.sq_quantize_weights(FAKE, BF16, r, c, None, FAKE, FAKE, None) == SQ_ERR_SHAPE
    assert lib.sq_w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 0, 4, 16, FAKE, F32, None) == SQ_ERR_SHAPE
    assert lib.sq_w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 133145, FAKE, F32, None) == SQ_ERR_SHAPE
    assert lib.sq_smooth_scales_from_absmax(FAKE, FAKE, 0, 0.5, FAKE, None) == SQ_ERR_SHAPE


def test_smooth_scales_maxima_outputs_optional(lib):
    """x_absmax and w_absmax may be NULL: the call gets past validation (the
    status is then that of the next check, here alpha) instead of SQ_ERR_NULL."""
    for xa, wa in ((None, FAKE), (FAKE, None), (None, None)):
        assert lib.sq_smooth_scales(FAKE, F32, 4, FAKE, BF16, 4, 8, 1.5, FAKE, xa, wa, None) == SQ_ERR_ALPHA
        assert lib.sq_smooth_scales(FAKE, F32, 0, FAKE, BF16, 4, 8, 0.5, FAKE, xa, wa, None) == SQ_ERR_SHAPE


def test_alpha_rejected(lib):
    for a in (-0.01, 1.01, float("nan"), float("inf")):
        assert lib.sq_smooth_scales_from_absmax(FAKE, FAKE, 8, a, FAKE, None) == SQ_ERR_ALPHA
        assert lib.sq_smooth_scales(FAKE, F32, 4, FAKE, F32, 4, 8, a, FAKE, FAKE, FAKE, None) == SQ_ERR_ALPHA


def test_dtypes_rejected(lib):
    assert lib.sq_col_absmax(FAKE, I32, 4, 4, FAKE, 0, None) == SQ_ERR_DTYPE
    assert lib.sq_quant_act(FAKE, 7, 4, 4, None, FAKE, FAKE, None) == SQ_ERR_DTYPE
    assert lib.sq_w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 16, FAKE, 5, None) == SQ_ERR_DTYPE
    # the linear layer produces floating-point outputs only
    assert lib.sq_w8a8_linear(FAKE, F32, None, FAKE, FAKE, 4, 4, 16, FAKE, I32, FAKE, 1 << 20,
                              None) == SQ_ERR_DTYPE


def test_workspace(lib):
    assert lib.sq_w8a8_linear_workspace_size(0, 4) == 0
    assert lib.sq_w8a8_linear_workspace_size(3, 100) == 512 + 256
    assert lib.sq_w8a8_linear_workspace_size(8192, 8192) == 8192 * 8192 + 8192 * 4
    # a product past size_t is reported as SIZE_MAX, not wrapped
    assert lib.sq_w8a8_linear_workspace_size(1 << 62, 8192) == 2 ** 64 - 1
    assert lib.sq_w8a8_linear_workspace_size(1 << 62, 1) == 2 ** 64 - 1
    need = lib.sq_w8a8_linear_workspace_size(16, 64)
    assert lib.sq_w8a8_linear(FAKE, F32, None, FAKE, FAKE, 16, 4, 64, FAKE, F32, FAKE, need - 1,
                              None) == SQ_ERR_WORKSPACE
    assert lib.sq_w8a8_linear(FAKE, F32, None, FAKE, FAKE, 16, 4, 64, FAKE, F32, None, need,
                              None) == SQ_ERR_WORKSPACE
    # workspace must be 256-byte aligned
    assert lib.sq_w8a8_linear(FAKE, F32, None, FAKE, FAKE, 16, 4, 64, FAKE, F32,
                              ctypes.c_void_p(0x1010), need, None) == SQ_ERR_WORKSPACE


def test_per_tensor_arguments(lib):
    assert lib.sq_act_absmax(FAKE, F32, 4, 4, None, None, 0, None) == SQ_ERR_NULL
    assert lib.sq_act_absmax(None, F32, 4, 4, None, FAKE, 0, None) == SQ_ERR_NULL
    assert lib.sq_act_absmax(FAKE, F32, 0, 4, None, FAKE, 0, None) == SQ_ERR_SHAPE
    assert lib.sq_act_absmax(FAKE, I32, 4, 4, None, FAKE, 0, None) == SQ_ERR_DTYPE
    assert lib.sq_quant_act_static(FAKE, F32, 4, 4, None, None, FAKE, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_quant_act_static(FAKE, BF16, 4, -2, None, FAKE, FAKE, FAKE, None) == SQ_ERR_SHAPE
    # the dynamic call validates everything before its first launch
    assert lib.sq_quant_act_per_tensor(FAKE, F32, 4, 4, None, FAKE, None, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_quant_act_per_tensor(FAKE, F32, 4, 4, None, FAKE, FAKE, None, None) == SQ_ERR_NULL


def test_norm_arguments(lib):
    assert lib.sq_fold_norm_gain(FAKE, None, 4, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_fold_norm_gain(FAKE, FAKE, 0, FAKE, None) == SQ_ERR_SHAPE
    ok = dict(X=FAKE, t=BF16, T=4, K=16, kind=0, g=FAKE, b=None, eps=1e-6, q=FAKE, xs=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.sq_norm_quant_act(a["X"], a["t"], a["T"], a["K"], a["kind"], a["g"], a["b"],
                                     a["eps"], a["q"], a["xs"], None, None, None)
    assert call(g=None) == SQ_ERR_NULL
    assert call(q=None) == SQ_ERR_NULL
    assert call(T=0) == SQ_ERR_SHAPE
    assert call(t=I32) == SQ_ERR_DTYPE
    assert call(kind=2) == SQ_ERR_ARG
    assert call(kind=0, b=FAKE) == SQ_ERR_ARG          # RMSNorm has no bias
    for eps in (-1e-6, float("nan"), float("inf")):
        assert call(eps=eps) == SQ_ERR_ARG


def test_decomp_arguments(lib):
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sq_decomp_select.argtypes = [P, I64, I64, P, P, P]
    lib.sq_decomp_prepare_weights.argtypes = [P, I, I64, I64, P, P, I64, P, P, P, P]
    lib.sq_decomp_quant_act.argtypes = [P, I, I64, I64, P, P, I64, P, P, P, P]
    lib.sq_decomp_gemm.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, I, P]
    assert lib.sq_decomp_select(FAKE, 16, 2, None, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_decomp_select(FAKE, 16, 17, FAKE, FAKE, None) == SQ_ERR_SHAPE
    assert lib.sq_decomp_select(FAKE, 16, -1, FAKE, FAKE, None) == SQ_ERR_SHAPE
    assert lib.sq_decomp_prepare_weights(FAKE, F32, 4, 16, FAKE, FAKE, 2, FAKE, FAKE, None, None) == SQ_ERR_NULL
    assert lib.sq_decomp_prepare_weights(FAKE, I32, 4, 16, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None) == SQ_ERR_DTYPE
    assert lib.sq_decomp_quant_act(FAKE, BF16, 4, 16, None, FAKE, 2, FAKE, FAKE, FAKE, None) == SQ_ERR_NULL
    assert lib.sq_decomp_quant_act(FAKE, BF16, 4, 16, FAKE, FAKE, 20, FAKE, FAKE, FAKE, None) == SQ_ERR_SHAPE
    # raw accumulators have no outlier term; outlier columns must be 16-byte aligned
    assert lib.sq_decomp_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 16, 2, FAKE, I32, None) == SQ_ERR_DTYPE
    assert lib.sq_decomp_gemm(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 4, 16, 2, FAKE, F32, None) == SQ_ERR_NULL
    assert lib.sq_decomp_gemm(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1004), FAKE, 4, 4, 16, 2, FAKE, F32,
                              None) == SQ_ERR_ARG


def test_noalloc_arguments(lib):
    """The no-allocation layer call validates on the host like sq_w8a8_linear
    and refuses problems whose codes and scales exceed its fixed scratch
    (32 MiB) before any launch."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sq_w8a8_linear_noalloc.argtypes = [P, I, P, P, P, I64, I64, I64, P, I, P]
    f = lib.sq_w8a8_linear_noalloc
    assert f(None, BF16, None, FAKE, FAKE, 4, 4, 16, FAKE, BF16, None) == SQ_ERR_NULL
    assert f(FAKE, BF16, None, FAKE, None, 4, 4, 16, FAKE, BF16, None) == SQ_ERR_NULL
    assert f(FAKE, BF16, None, FAKE, FAKE, 4, 4, 16, FAKE, I32, None) == SQ_ERR_DTYPE
    assert f(FAKE, BF16, None, FAKE, FAKE, 0, 4, 16, FAKE, BF16, None) == SQ_ERR_SHAPE
    # 8192 x 8192 codes (64 MiB) and one token past 32 MiB of codes
    assert f(FAKE, BF16, None, FAKE, FAKE, 8192, 8192, 8192, FAKE, BF16, None) == SQ_ERR_SCRATCH
    assert f(FAKE, BF16, None, FAKE, FAKE, 4097, 4, 8192, FAKE, BF16, None) == SQ_ERR_SCRATCH
    # T * K past 2^64 must not wrap into the scratch size
    assert f(FAKE, BF16, None, FAKE, FAKE, (1 << 63) - 1, 4, 8192, FAKE, BF16, None) == SQ_ERR_SCRATCH
    assert f(FAKE, BF16, None, FAKE, FAKE, 1 << 51, 4, 8192, FAKE, BF16, None) == SQ_ERR_SCRATCH
    assert b"SQ_ERR_SCRATCH" in lib.sq_status_string(SQ_ERR_SCRATCH)
