"""Launch trace: with SQ_TRACE=1 every kernel launch of the library writes one
line to stderr naming the kernel and its configuration; without it, nothing."""
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _layer(sq, T, N, K, rng):
    X = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    s, _, _ = sq.sq_smooth_scales(X, W, 0.5)
    Wq, ws = sq.sq_quantize_weights(W, s)
    return X, s, Wq, ws


def test_trace_lines(sq, capfd):
    rng = np.random.default_rng(5)
    prefill = _layer(sq, 300, 512, 1024, rng)
    decode = _layer(sq, 16, 1024, 2048, rng)
    torch.cuda.synchronize()
    capfd.readouterr()
    old = os.environ.get("SQ_TRACE")
    os.environ["SQ_TRACE"] = "1"
    try:
        for X, s, Wq, ws in (prefill, decode):
            sq.sq_w8a8_linear(X, s, Wq, ws)
        torch.cuda.synchronize()
        err = capfd.readouterr().err.splitlines()
    finally:
        if old is None:
            del os.environ["SQ_TRACE"]
        else:
            os.environ["SQ_TRACE"] = old
    lines = [l for l in err if l.startswith("sq: ")]
    # one quantiser launch and one GEMM launch per layer call, in call order
    kinds = [l.split()[1] for l in lines]
    assert kinds == ["quant_rows", "gemm_i8_mfma", "quant_rows", "gemv_i8_mfma"], lines
    assert "T 300 N 512 K 1024" in lines[1] and "out bf16" in lines[1]
    assert "T 16 N 1024 K 2048" in lines[3]
    assert "R 300 K 1024" in lines[0] and "R 16 K 2048" in lines[2]
    # the 1 KB-segment decode form: wide layer, K a multiple of 4096
    wide = _layer(sq, 16, 16384, 8192, rng)
    torch.cuda.synchronize()
    capfd.readouterr()
    os.environ["SQ_TRACE"] = "1"
    try:
        sq.sq_w8a8_linear(*wide)
        torch.cuda.synchronize()
        err = capfd.readouterr().err.splitlines()
    finally:
        if old is None:
            del os.environ["SQ_TRACE"]
        else:
            os.environ["SQ_TRACE"] = old
    lines = [l for l in err if l.startswith("sq: ")]
    assert [l.split()[1] for l in lines] == ["quant_rows", "gemv_seg_i8_mfma"], lines
    assert "T 16 N 16384 K 8192" in lines[1]
    # switched off again: no lines
    X, s, Wq, ws = prefill
    sq.sq_w8a8_linear(X, s, Wq, ws)
    torch.cuda.synchronize()
    assert not [l for l in capfd.readouterr().err.splitlines() if l.startswith("sq: ")]
