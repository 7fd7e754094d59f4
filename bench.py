"""Throughput of the SmoothQuant W8A8 linear layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-decode]

One step is one pass of the whole path over one batch of synthetic input, all
through libsq.so on the current HIP stream:
    sq_smooth_scales     column absmax of the statistics batch and of W, then s
    sq_quantize_weights  W diag(s) -> per-output-channel int8
    sq_quant_act         X diag(s)^-1 -> per-token int8     (sq_w8a8_linear's 1st launch)
    sq_w8a8_gemm         int8 GEMM + dequant epilogue       (sq_w8a8_linear's 2nd launch)
`value` is 2*T*N*K / (time per step) in TOPS, with inputs resident in HBM.  Each
call is bracketed by HIP events on the same stream, so the per-kernel averages
come from inside the timed region.  Default workload: heavy-outlier prefill,
X bf16 [8192 x 8192] (30% outlier channels), W [8192 x 8192], alpha 0.75, bf16 out.

Also printed in the same JSON line: the GEMM's roofline fraction against the
dense INT8 MFMA peak, the quantiser's HBM rate, the decode-shaped GEMM
(16 x 28672 x 8192) HBM rate with three weight copies rotated so that every
launch streams from HBM rather than the 256 MB Infinity Cache, and the CPU
oracle timed on a bounded token sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 linear TOPS incl. per-token quant (prefill); HBM GB/s (quant, decode GEMM)"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published


def _gemm_bytes(T, N, K, out_bytes):
    """Algorithmic bytes of one GEMM launch: Wq, w_scale, Xq, x_scale in; Y out."""
    return N * K + 4 * N + T * K + 4 * T + out_bytes * T * N


def _quant_bytes(T, K, in_bytes):
    """Algorithmic bytes of one activation-quantiser launch: X and s in; codes and scales out."""
    return in_bytes * T * K + 4 * K + T * K + 4 * T


def _omp_threads():
    try:
        import ctypes
        return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(w, target_s=12.0):
    """The oracle as it stands, on a prefix of the workload's tokens: statistics,
    smoothing factors and weight quantisation in full, then quantisation, integer
    GEMM, epilogue and bf16 rounding for `tokens` tokens.  Throughput in TOPS of
    the sample's 2*tokens*N*K over the wall time of all of it."""
    import oracle as O
    O.build()

    def offline():
        xa = O.col_absmax(w.stats_source)
        wa = O.col_absmax(w.W)
        s = O.smooth_scales(xa, wa, w.alpha)
        Wq, ws = O.quantize_weights(w.W, s)
        return s, Wq, ws

    def runtime(s, Wq, ws, tokens):
        Xq, xs = O.quant_act(w.X[:tokens], s)
        y = O.dequant(O.int_gemm(Xq, Wq), xs, ws)
        if w.y_dtype == "bf16":
            O.to_bf16(y)

    s, Wq, ws = offline()
    probe = min(8, w.T)
    t0 = time.perf_counter()
    runtime(s, Wq, ws, probe)
    per_token = (time.perf_counter() - t0) / probe
    tokens = int(max(1, min(w.T, target_s / max(per_token, 1e-6))))
    t0 = time.perf_counter()
    s, Wq, ws = offline()
    runtime(s, Wq, ws, tokens)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * tokens * w.N * w.K / dt / 1e12, "unit": "TOPS", "cores": _omp_threads(),
            "kind": "oracle",
            "sample": f"first {tokens} of {w.T} tokens; column maxima, smoothing factors and weight "
                      f"quantisation over the full tensors; {dt:.1f} s wall"}


def decode_measure(sq, torch, reps=30):
    """Decode-shaped GEMM rate: 3 copies of the int8 weights (3 x 235 MB, more
    than the 256 MB Infinity Cache) used in turn, one event pair per launch."""
    import workloads as WL
    w = WL.make("decode_t16_k8192_n28672")
    dev = torch.device("cuda")
    X = torch.from_numpy(w.X).to(torch.bfloat16).to(dev)
    W = torch.from_numpy(w.W).to(dev)
    Xc = torch.from_numpy(w.X_calib).to(torch.bfloat16).to(dev)
    s, _, _ = sq.sq_smooth_scales(Xc, W, w.alpha)
    Wq, ws = sq.sq_quantize_weights(W, s)
    del W
    copies = [Wq] + [Wq.clone() for _ in range(2)]
    Xq, xs = sq.sq_quant_act(X, s)
    Y = torch.empty((w.T, w.N), dtype=torch.bfloat16, device=dev)
    for i in range(6):
        sq.sq_w8a8_gemm(Xq, xs, copies[i % 3], ws, Y=Y)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        sq.sq_w8a8_gemm(Xq, xs, copies[i % 3], ws, Y=Y)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    byts = _gemm_bytes(w.T, w.N, w.K, 2)
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": w.name, "T": w.T, "N": w.N, "K": w.K, "us": ms * 1e3, "GB/s": gbs,
            "frac_hbm": gbs / PEAK_HBM_GBS, "bytes": byts, "weight_copies_rotated": 3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="heavy_t8192_k8192_n8192")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU only: the path has no multi-GPU mode "
              "(no sharding or collectives are built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as WL
    import w8a8_quantized_amd as sq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WL.make(args.workload)
    T, N, K = w.T, w.N, w.K
    xdt = torch.bfloat16 if w.x_dtype == "bf16" else torch.float32
    ydt = torch.bfloat16 if w.y_dtype == "bf16" else torch.float32
    X = torch.from_numpy(w.X).to(xdt).to(dev)
    Xs = X if w.X_calib is None else torch.from_numpy(w.X_calib).to(xdt).to(dev)
    W = torch.from_numpy(w.W).to(dev)
    s = torch.empty(K, device=dev)
    xa = torch.empty(K, device=dev)
    wa = torch.empty(K, device=dev)
    Wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    ws = torch.empty(N, device=dev)
    Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    xs = torch.empty(T, device=dev)
    Y = torch.empty((T, N), dtype=ydt, device=dev)

    def step(ev=None):
        if ev: ev[0].record()
        sq.sq_smooth_scales(Xs, W, w.alpha, s=s, x_absmax=xa, w_absmax=wa)
        if ev: ev[1].record()
        sq.sq_quantize_weights(W, s, Wq=Wq, w_scale=ws)
        if ev: ev[2].record()
        sq.sq_quant_act(X, s, Xq=Xq, x_scale=xs)
        if ev: ev[3].record()
        sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=ydt, Y=Y)
        if ev: ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    ms_step = wall * 1e3 / args.steps

    def avg(i):
        return float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))

    t_smooth, t_wq, t_quant, t_gemm = avg(0), avg(1), avg(2), avg(3)
    ops = 2.0 * T * N * K
    ob = 2 if ydt == torch.bfloat16 else 4
    ib = 2 if xdt == torch.bfloat16 else 4
    gemm_tops = ops / (t_gemm * 1e-3) / 1e12
    qbytes = _quant_bytes(T, K, ib)
    out = {
        "metric": METRIC,
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "N": N, "K": K, "alpha": w.alpha,
                   "x_dtype": w.x_dtype, "w_dtype": "f32", "y_dtype": w.y_dtype,
                   "stats_tokens": int(Xs.shape[0]),
                   "step": "smooth_scales + quantize_weights + quant_act + w8a8_gemm"},
        "roofline": {"kernel": "gemm_i8_mfma (sq_w8a8_gemm)", "bound": "mfma",
                     "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": gemm_tops / PEAK_INT8_TOPS, "traffic": None,
                     "per_launch_ops": ops, "avg_launch_ms": t_gemm},
        "breakdown_ms": {"smooth_scales": t_smooth, "quantize_weights": t_wq, "quant_act": t_quant,
                         "w8a8_gemm": t_gemm},
        "linear_tops": ops / ((t_quant + t_gemm) * 1e-3) / 1e12,
        "quant_act": {"GB/s": qbytes / (t_quant * 1e-3) / 1e9,
                      "frac_hbm": qbytes / (t_quant * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": qbytes},
    }
    if not args.no_decode:
        del X, Xs, W, Wq, Xq, Y
        torch.cuda.empty_cache()
        out["decode_gemm"] = decode_measure(sq, torch)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
