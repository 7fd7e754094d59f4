"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

No call allocates device memory and the running maxima are cleared by a fill
kernel, so the calls can be captured and replayed.  Each graph is replayed
several times with new inputs copied into its static buffers, eager work and
synchronisations between the replays, and every replay is compared bit for bit
with an eager call on the same inputs.
"""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import DEV, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import w8a8_quantized_amd as m   # raises if libsq.so is missing: no fallback
    assert torch.cuda.is_available()
    return m


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _draw(rng, T, K, scale=1.0):
    X = rng.standard_normal((T, K)).astype(np.float32) * scale
    X[:, rng.choice(K, 3, replace=False)] *= 40
    return torch.from_numpy(X).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("T,N,K", [(300, 384, 512), (16, 512, 1024), (16, 16448, 8192)])
def test_linear_graph_replays(sq, T, N, K):
    """sq_w8a8_linear (quantiser + GEMM, or the decode GEMM at T <= 32)."""
    rng = np.random.default_rng(T + N + K)
    w = WL.page_tiny_fixture(seed=11, T=T, N=N, K=K)
    W = torch.from_numpy(w.W).to(DEV)
    s, _, _ = sq.sq_smooth_scales(_draw(rng, T, K), W, 0.5)
    Wq, ws = sq.sq_quantize_weights(W, s)
    X_in = _draw(rng, T, K)
    Y_g = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    buf = torch.empty(sq.sq_w8a8_linear_workspace_size(T, K), dtype=torch.uint8, device=DEV)
    g = _capture(lambda: sq.sq_w8a8_linear(X_in, s, Wq, ws, Y=Y_g, workspace=buf))
    for r in range(4):
        X = _draw(rng, T, K, scale=1.0 + r)
        X_in.copy_(X)
        g.replay()
        torch.cuda.synchronize()
        want = sq.sq_w8a8_linear(X, s, Wq, ws)   # eager, own buffers
        torch.cuda.synchronize()
        assert np.array_equal(host(Y_g), host(want)), f"replay {r}"


@pytest.mark.parametrize("T,N,K", [(300, 384, 512), (16, 512, 1024)])
def test_noalloc_linear_graph_replays(sq, T, N, K):
    """sq_w8a8_linear_noalloc, the entry point for callers that cannot allocate
    (its workspace is the library's fixed per-GPU scratch): captured, replayed
    with new inputs, each replay equal to the workspace call."""
    rng = np.random.default_rng(7 * T + N + K)
    w = WL.page_tiny_fixture(seed=13, T=T, N=N, K=K)
    W = torch.from_numpy(w.W).to(DEV)
    s, _, _ = sq.sq_smooth_scales(_draw(rng, T, K), W, 0.5)
    Wq, ws = sq.sq_quantize_weights(W, s)
    X_in = _draw(rng, T, K)
    Y_g = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    g = _capture(lambda: sq.sq_w8a8_linear_noalloc(X_in, s, Wq, ws, Y_g))
    for r in range(4):
        X = _draw(rng, T, K, scale=1.0 + r)
        X_in.copy_(X)
        g.replay()
        torch.cuda.synchronize()
        want = sq.sq_w8a8_linear(X, s, Wq, ws)   # eager, caller workspace
        torch.cuda.synchronize()
        assert np.array_equal(host(Y_g), host(want)), f"replay {r}"


def test_smooth_scales_graph_replays(sq):
    """The statistics pass: zero fill, fused column maxima, factors."""
    rng = np.random.default_rng(3)
    T, N, K = 200, 300, 1024
    X_in = _draw(rng, T, K)
    W_in = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    s = torch.empty(K, device=DEV)
    xa = torch.empty(K, device=DEV)
    wa = torch.empty(K, device=DEV)
    g = _capture(lambda: sq.sq_smooth_scales(X_in, W_in, 0.5, s=s, x_absmax=xa, w_absmax=wa))
    for r in range(4):
        # smaller values after larger ones: a stale maximum would survive a missing clear
        X = _draw(rng, T, K, scale=4.0 - r)
        W = torch.from_numpy((rng.standard_normal((N, K)) * (0.08 - 0.02 * r)).astype(np.float32)).to(DEV)
        X_in.copy_(X)
        W_in.copy_(W)
        g.replay()
        torch.cuda.synchronize()
        s_e, xa_e, wa_e = sq.sq_smooth_scales(X, W, 0.5)
        torch.cuda.synchronize()
        assert np.array_equal(host(xa), host(xa_e)) and np.array_equal(host(wa), host(wa_e)), f"replay {r}"
        assert np.array_equal(host(s), host(s_e)), f"replay {r}"


@pytest.mark.parametrize("T,N,K,n_o", [(16, 640, 512, 9), (16, 16448, 8192, 41)])
def test_decomp_gemm_graph_replays(sq, T, N, K, n_o):
    """The decode GEMM with the outlier term (dynamic LDS for the outlier
    operands), in the 256-byte and the 1 KB-segment form."""
    rng = np.random.default_rng(5)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).to(DEV)
    a = torch.from_numpy(rng.uniform(0, 1, K).astype(np.float32)).to(DEV)
    idx, mask = sq.sq_decomp_select(a, n_o)
    Wq, ws, Wo = sq.sq_decomp_prepare_weights(W, mask, idx)
    X_in = _draw(rng, T, K)
    Xq, xs, Xo = sq.sq_decomp_quant_act(X_in, mask, idx)
    Y_g = torch.empty((T, N), dtype=torch.float32, device=DEV)

    def layer():
        sq.sq_decomp_quant_act(X_in, mask, idx, Xq=Xq, x_scale=xs, X_out=Xo)
        sq.sq_decomp_gemm(Xq, xs, Wq, ws, Xo, Wo, out_dtype=torch.float32, Y=Y_g)

    g = _capture(layer)
    for r in range(4):
        X = _draw(rng, T, K, scale=1.0 + r)
        X_in.copy_(X)
        g.replay()
        torch.cuda.synchronize()
        Xq_e, xs_e, Xo_e = sq.sq_decomp_quant_act(X, mask, idx)
        want = sq.sq_decomp_gemm(Xq_e, xs_e, Wq, ws, Xo_e, Wo, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(host(Y_g), host(want)), f"replay {r}"


@pytest.mark.parametrize("T,N,K", [(2100, 8200, 208), (300, 520, 336), (16, 640, 512), (16, 16448, 8192)])
def test_fp8_gemm_graph_replays(sq, T, N, K):
    """sq_fp8_gemm (persistent 256x256 form, 64x64 tiles, both decode forms) with
    its FP8 operands copied into the captured buffers before each replay."""
    rng = np.random.default_rng(T + N + K)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).to(DEV)
    Wq, ws = sq.sq_quantize_weights_fp8(W)
    X_in = _draw(rng, T, K)
    Xq_in, xs_in = sq.sq_quant_act_fp8(X_in)
    Y_g = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    g = _capture(lambda: sq.sq_fp8_gemm(Xq_in, xs_in, Wq, ws, Y=Y_g))
    for r in range(4):
        Xq, xs = sq.sq_quant_act_fp8(_draw(rng, T, K, scale=1.0 + r))
        Xq_in.copy_(Xq)
        xs_in.copy_(xs)
        g.replay()
        torch.cuda.synchronize()
        want = sq.sq_fp8_gemm(Xq, xs, Wq, ws)   # eager, own output
        torch.cuda.synchronize()
        assert np.array_equal(host(Y_g), host(want)), f"replay {r}"
