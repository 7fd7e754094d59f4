"""Throughput of the SmoothQuant W8A8 linear layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-decode]
    python bench.py --configs      # per-configuration figures, one JSON object per line

One step is one pass of the whole path over one batch of synthetic input, all
through libsq.so on the current HIP stream:
    sq_smooth_scales     column absmax of the statistics batch and of W, then s
    sq_quantize_weights  W diag(s) -> per-output-channel int8
    sq_quant_act         X diag(s)^-1 -> per-token int8     (sq_w8a8_linear's 1st launch)
    sq_w8a8_gemm         int8 GEMM + dequant epilogue       (sq_w8a8_linear's 2nd launch)
`value` is 2*T*N*K / (time per step) in TOPS, with inputs resident in HBM.  In
the timed region one pair of HIP events per step, on the same stream, brackets
the GEMM (the dominant kernel) for the roofline figure; the per-call breakdown
is measured before the warm-up, with batched back-to-back launches.  Default workload: heavy-outlier prefill,
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
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published


def _gemm_bytes(T, N, K, out_bytes):
    """Algorithmic bytes of one GEMM launch: Wq, w_scale, Xq, x_scale in; Y out."""
    return N * K + 4 * N + T * K + 4 * T + out_bytes * T * N


def _quant_bytes(T, K, in_bytes):
    """Algorithmic bytes of one activation-quantiser launch: X and s in; codes and scales out."""
    return in_bytes * T * K + 4 * K + T * K + 4 * T


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_pmc_heavy_t8192_and_decode_t16.md")


def _gemm_traffic(workload):
    """Memory-side bytes (read + written) of one GEMM launch from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, or None when that summary is for
    another workload or the GEMM source has changed since it was taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_SUMMARY).read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in lines if ": " in l and not l.startswith(("|", " ", "#")))
    src = b"".join(open(os.path.join(ROOT, "w8a8_quantized_amd", "csrc", f), "rb").read()
                   for f in ("k_gemm.hip", "common.h"))
    if kv.get("workload") != workload or kv.get("gemm_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return float(kv["gemm_traffic_bytes_per_launch"])


def _rate(nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us": ms * 1e3, "bytes": nbytes, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}


def _omp_threads():
    try:
        import ctypes
        return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s=20.0, runs=3):
    """The oracle as it stands, on a prefix of the workload's tokens: statistics,
    smoothing factors and weight quantisation in full, then quantisation, integer
    GEMM, epilogue and bf16 rounding for `tokens` tokens.  Throughput in TOPS of
    the sample's 2*tokens*N*K over the wall time of all of it; the median of
    `runs` runs, each sized for about target_s / runs seconds."""
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
    probe = min(64, w.T)   # enough rows for the OpenMP loops to spread over the cores
    t0 = time.perf_counter()
    runtime(s, Wq, ws, probe)
    per_token = (time.perf_counter() - t0) / probe
    tokens = int(max(1, min(w.T, target_s / runs / max(per_token, 1e-6))))
    rates, walls = [], []
    for _ in range(runs):
        t0 = time.perf_counter()
        s, Wq, ws = offline()
        runtime(s, Wq, ws, tokens)
        dt = time.perf_counter() - t0
        walls.append(dt)
        rates.append(2.0 * tokens * w.N * w.K / dt / 1e12)
    return {"value": float(np.median(rates)), "unit": "TOPS", "cores": _omp_threads(),
            "cpu_model": _cpu_model(), "runs": runs, "kind": "oracle",
            "sample": f"first {tokens} of {w.T} tokens; column maxima, smoothing factors and weight "
                      f"quantisation over the full tensors; median of {runs} runs of "
                      f"{', '.join(f'{d:.1f}' for d in walls)} s wall"}


def decode_measure(sq, torch, reps=30, placements=3):
    """Decode-shaped GEMM rate: 3 copies of the int8 weights (3 x 235 MB, more
    than the 256 MB Infinity Cache) used in turn; `reps` launches back to back
    between two events.  The rate depends on where the weights land in memory
    (fresh allocations of the same copies differ by up to ~17%), so the copies
    are allocated `placements` times and the median is reported, with every
    value."""
    import workloads as WL
    w = WL.make("decode_t16_k8192_n28672")
    dev = torch.device("cuda")
    X = torch.from_numpy(w.X).to(torch.bfloat16).to(dev)
    W = torch.from_numpy(w.W).to(dev)
    Xc = torch.from_numpy(w.X_calib).to(torch.bfloat16).to(dev)
    s, _, _ = sq.sq_smooth_scales(Xc, W, w.alpha)
    Wq, ws = sq.sq_quantize_weights(W, s)
    Wq8, ws8 = sq.sq_quantize_weights_fp8(W, s)
    del W
    torch.cuda.empty_cache()
    Xq, xs = sq.sq_quant_act(X, s)
    Xq8, xs8 = sq.sq_quant_act_fp8(X, s)
    Y = torch.empty((w.T, w.N), dtype=torch.bfloat16, device=dev)

    def per_launch(fn, cps):
        for i in range(6):
            fn(cps[i % 3])
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)   # keeps the GPU busy while the launches are queued
        a.record()
        for i in range(reps):
            fn(cps[i % 3])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    runs, runs8, held = [], [], []
    for _ in range(placements):
        copies = [Wq.clone() for _ in range(3)]       # each copy in an allocation of its own
        copies8 = [Wq8.clone() for _ in range(3)]
        runs.append(per_launch(lambda wq: sq.sq_w8a8_gemm(Xq, xs, wq, ws, Y=Y), copies))
        runs8.append(per_launch(lambda wq: sq.sq_fp8_gemm(Xq8, xs8, wq, ws8, Y=Y), copies8))
        held.append((copies, copies8))                 # kept, so the next set lands elsewhere
    ms, ms8 = float(np.median(runs)), float(np.median(runs8))
    byts = _gemm_bytes(w.T, w.N, w.K, 2)
    gbs, gbs8 = byts / (ms * 1e-3) / 1e9, byts / (ms8 * 1e-3) / 1e9
    del held
    torch.cuda.empty_cache()
    return {"workload": w.name, "T": w.T, "N": w.N, "K": w.K, "us": ms * 1e3, "GB/s": gbs,
            "frac_hbm": gbs / PEAK_HBM_GBS, "bytes": byts, "weight_copies_rotated": 3,
            "us_per_placement": [round(x * 1e3, 2) for x in runs],
            "placements": f"median over {placements} allocations of the three weight copies",
            "fp8": {"us": ms8 * 1e3, "GB/s": gbs8, "frac_hbm": gbs8 / PEAK_HBM_GBS,
                    "us_per_placement": [round(x * 1e3, 2) for x in runs8]}}


def _time_calls(torch, fn, copies, reps=20):
    """Per-call time (ms) of `reps` back-to-back calls cycling through `copies`,
    queued behind a GPU-side wait so that host launch time is not measured."""
    for i in range(3):
        fn(copies[i % len(copies)])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    a.record()
    for i in range(reps):
        fn(copies[i % len(copies)])
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def decomp_measure(sq, torch):
    """Mixed-precision decomposition on the two workloads with planted outlier
    channels (their count taken as the static set, chosen from the calibration
    draw), next to the smoothed per-token path on the same shapes."""
    import workloads as WL
    dev = torch.device("cuda")
    out = {}
    for name, n_o in (("prefill_t2048_k4096_n16384", 8), ("decode_t16_k8192_n28672", 41)):
        w = WL.make(name)
        T, N, K = w.T, w.N, w.K
        X = torch.from_numpy(w.X).to(torch.bfloat16).to(dev)
        Xc = torch.from_numpy(w.X_calib).to(torch.bfloat16).to(dev)
        W = torch.from_numpy(w.W).to(dev)
        idx, mask = sq.sq_decomp_select(sq.sq_col_absmax(Xc), n_o)
        Wq_d, ws_d, Wo = sq.sq_decomp_prepare_weights(W, mask, idx)
        s, _, _ = sq.sq_smooth_scales(Xc, W, w.alpha)
        Wq_s, ws_s = sq.sq_quantize_weights(W, s)
        del W
        torch.cuda.empty_cache()
        # decode: rotate three copies of the weights (more than the Infinity Cache)
        nc = 3 if T <= 64 else 1
        Wd = [Wq_d] + [Wq_d.clone() for _ in range(nc - 1)]
        Ws = [Wq_s] + [Wq_s.clone() for _ in range(nc - 1)]
        Xq_d, xs_d, Xo = sq.sq_decomp_quant_act(X, mask, idx)
        Xq_s, xs_s = sq.sq_quant_act(X, s)
        Y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        t_qd = _time_calls(torch, lambda _: sq.sq_decomp_quant_act(X, mask, idx, Xq=Xq_d, x_scale=xs_d, X_out=Xo), [None])
        t_qs = _time_calls(torch, lambda _: sq.sq_quant_act(X, s, Xq=Xq_s, x_scale=xs_s), [None])
        t_gd = _time_calls(torch, lambda wq: sq.sq_decomp_gemm(Xq_d, xs_d, wq, ws_d, Xo, Wo, Y=Y), Wd)
        t_gs = _time_calls(torch, lambda wq: sq.sq_w8a8_gemm(Xq_s, xs_s, wq, ws_s, Y=Y), Ws)
        ops = 2.0 * T * N * K
        out[name] = {"n_outliers": n_o,
                     "decomp_quant_act_us": t_qd * 1e3, "smooth_quant_act_us": t_qs * 1e3,
                     "decomp_gemm_us": t_gd * 1e3, "smooth_gemm_us": t_gs * 1e3,
                     "decomp_linear_TOPS": ops / ((t_qd + t_gd) * 1e-3) / 1e12,
                     "smooth_linear_TOPS": ops / ((t_qs + t_gs) * 1e-3) / 1e12}
        del Wd, Ws, Wq_d, Wq_s, X, Xc, Y
        torch.cuda.empty_cache()
    return out


def configs_report(sq, torch):
    """Per-configuration figures (one JSON object per line, not the contract
    line): the run-time layer (sq_quant_act + sq_w8a8_gemm) on each named
    workload with its own smoothing factors, timed as 7 batches of 20
    back-to-back calls (median and 10th / 90th percentile of the batch means).
    The large inputs are rotated over three copies when they exceed the
    Infinity Cache."""
    import workloads as WL
    dev = torch.device("cuda")
    for name in WL.WORKLOADS:
        w = WL.make(name)
        T, N, K = w.T, w.N, w.K
        xdt = torch.bfloat16 if w.x_dtype == "bf16" else torch.float32
        ydt = torch.bfloat16 if w.y_dtype == "bf16" else torch.float32
        X = torch.from_numpy(w.X).to(xdt).to(dev)
        Xs = X if w.X_calib is None else torch.from_numpy(w.X_calib).to(xdt).to(dev)
        W = torch.from_numpy(w.W).to(dev)
        s, _, _ = sq.sq_smooth_scales(Xs, W, w.alpha)
        Wq, ws = sq.sq_quantize_weights(W, s)
        del W
        torch.cuda.empty_cache()
        Xq, xs = sq.sq_quant_act(X, s)
        Y = torch.empty((T, N), dtype=ydt, device=dev)
        big = N * K > 128 << 20
        Wc = [Wq] + ([Wq.clone() for _ in range(2)] if big else [])
        Xc = [X] + ([X.clone() for _ in range(2)] if T * K * X.element_size() > 128 << 20 else [])
        # 7 batches of 20 calls each; median, 10th and 90th percentile of the
        # per-call means
        qs = [_time_calls(torch, lambda x_: sq.sq_quant_act(x_, s, Xq=Xq, x_scale=xs), Xc) for _ in range(7)]
        gs = [_time_calls(torch, lambda wq: sq.sq_w8a8_gemm(Xq, xs, wq, ws, out_dtype=ydt, Y=Y), Wc)
              for _ in range(7)]
        t_q, t_g = float(np.median(qs)), float(np.median(gs))
        pct = lambda v: [round(float(np.percentile(v, q)) * 1e3, 2) for q in (10, 50, 90)]
        ops = 2.0 * T * N * K
        gb = _gemm_bytes(T, N, K, 2 if ydt == torch.bfloat16 else 4)
        qb = _quant_bytes(T, K, X.element_size())
        print(json.dumps({"workload": name, "T": T, "N": N, "K": K, "alpha": w.alpha,
                          "linear_TOPS": ops / ((t_q + t_g) * 1e-3) / 1e12,
                          "gemm_us": t_g * 1e3, "gemm_TOPS": ops / (t_g * 1e-3) / 1e12,
                          "gemm_frac_int8_peak": ops / (t_g * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                          "gemm_GB/s": gb / (t_g * 1e-3) / 1e9,
                          "gemm_frac_hbm": gb / (t_g * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "quant_us": t_q * 1e3, "quant_GB/s": qb / (t_q * 1e-3) / 1e9,
                          "quant_frac_hbm": qb / (t_q * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "gemm_us_p10_p50_p90": pct(gs), "quant_us_p10_p50_p90": pct(qs),
                          "batches": "7 x 20 calls", "copies_rotated": len(Wc)}), flush=True)
        del X, Xs, Wq, Xq, Y, Wc, Xc
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30)   # the clocks settle within ~20 ms of load
    ap.add_argument("--workload", default="heavy_t8192_k8192_n8192")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="print per-configuration figures for every named workload instead")
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
    if args.configs:
        configs_report(sq, torch)
        return
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
        sq.sq_smooth_scales(Xs, W, w.alpha, s=s, x_absmax=xa, w_absmax=wa)
        sq.sq_quantize_weights(W, s, Wq=Wq, w_scale=ws)
        sq.sq_quant_act(X, s, Xq=Xq, x_scale=xs)
        if ev: ev[0].record()
        sq.sq_w8a8_gemm(Xq, xs, Wq, ws, out_dtype=ydt, Y=Y)
        if ev: ev[1].record()

    # Per-call figures first, then the timed steps: the GPU runs at a lower clock
    # for its first ~20 ms of load, and measured after that settling (rather than
    # right after the warm-up steps) the step and its GEMM reflect the sustained
    # rate.  Decode-shaped and decomposition figures (their own workloads) come
    # first, then this workload's entry points, each launched `reps` times back
    # to back between two events, cycling through 3 copies of its large input so
    # that every launch reads from HBM rather than from the 256 MB Infinity
    # Cache.  The int8 GEMM of this workload is not among them: its per-launch
    # time comes from the timed region itself.
    extra = {}
    if not args.no_decode:
        extra["decode_gemm"] = decode_measure(sq, torch)
        extra["decomposition"] = decomp_measure(sq, torch)
        torch.cuda.empty_cache()

    def batched(fn, copies, reps=20, batches=3):
        """Median over `batches` of the per-call time of `reps` back-to-back
        calls, each batch queued behind a GPU-side wait (host launch time not
        measured)."""
        return float(np.median([_time_calls(torch, fn, copies, reps) for _ in range(batches)]))

    step()
    Wc = [W, W.clone(), W.clone()]
    Xc = [X, X.clone(), X.clone()]
    # FP8 E4M3 variant of the same layer: quantisers and the FP8 matrix-core GEMM
    Wq8, ws8 = sq.sq_quantize_weights_fp8(W, s)
    Xq8, xs8 = sq.sq_quant_act_fp8(X, s)
    t_q8 = batched(lambda x_: sq.sq_quant_act_fp8(x_, s, Xq=Xq8, x_scale=xs8), Xc)
    # per-tensor activation scales: the range reduction alone, the static-range
    # quantiser (range from the first 512 tokens, as a calibration would give),
    # and the dynamic per-tensor quantiser (reduction + quantiser)
    amax_buf = torch.empty(1, device=dev)
    clip_buf = sq.sq_act_absmax(X[:512], s)
    t_tabs = batched(lambda x_: sq.sq_act_absmax(x_, s, amax=amax_buf), Xc)
    t_qstat = batched(lambda x_: sq.sq_quant_act_static(x_, s, clip_buf, Xq=Xq, x_scale=xs), Xc)
    t_qpt = batched(lambda x_: sq.sq_quant_act_per_tensor(x_, s, amax=amax_buf, Xq=Xq, x_scale=xs), Xc)
    # the producer in front of the layer: RMSNorm (gain folded with s) + per-token int8
    gen = torch.Generator(device=dev).manual_seed(7)
    gain = 1.0 + 0.2 * torch.randn(K, device=dev, generator=gen)
    gfold = sq.sq_fold_norm_gain(gain, s)
    m_buf, r_buf = torch.empty(T, device=dev), torch.empty(T, device=dev)
    t_norm = batched(lambda x_: sq.sq_norm_quant_act(x_, "rms", gfold, Xq=Xq, x_scale=xs, mean=m_buf,
                                                     rstd=r_buf), Xc)
    t_smooth = batched(lambda w_: sq.sq_smooth_scales(Xs, w_, w.alpha, s=s, x_absmax=xa, w_absmax=wa), Wc)
    t_wq = batched(lambda w_: sq.sq_quantize_weights(w_, s, Wq=Wq, w_scale=ws), Wc)
    t_quant = batched(lambda x_: sq.sq_quant_act(x_, s, Xq=Xq, x_scale=xs), Xc)
    # The FP8 GEMM goes last: the GPU's power management needs several
    # milliseconds of matrix-core load to settle (coming from memory-bound
    # kernels, the 8192^3 int8 GEMM first runs at 530-555 us and takes ~15 steps
    # to return to ~455 us), so ending the per-call figures with a GEMM leaves
    # the timed steps at the sustained rate.
    t_g8 = batched(lambda _: sq.sq_fp8_gemm(Xq8, xs8, Wq8, ws8, out_dtype=ydt, Y=Y), [None])
    del Wc, Xc, Wq8, Xq8

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps.  An event pair on the stream every call is
    # enqueued on brackets the GEMM (the dominant kernel) in every EVERY-th step:
    # each event record lets the queue drain before the next launch (~7 us of
    # idle GPU per pair), so bracketing every step would slow the step ~1%.  The
    # events are created (recorded once) before the timed region.
    EVERY = 4
    timed = [i for i in range(args.steps) if i % EVERY == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in timed}
    for e in evs.values():
        e[0].record()
        e[1].record()
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    ms_step = wall * 1e3 / args.steps
    launch_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in timed])
    t_gemm = float(np.mean(launch_ms))

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
                     "frac": gemm_tops / PEAK_INT8_TOPS, "traffic": _gemm_traffic(w.name),
                     "traffic_unit": "bytes per launch (memory side, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "per_launch_ops": ops, "avg_launch_ms": t_gemm, "timed_launches": len(timed),
                     "launch_ms_p10_p50_p90": [float(np.percentile(launch_ms, q)) for q in (10, 50, 90)]},
        "breakdown_ms_batched": {"smooth_scales": t_smooth, "quantize_weights": t_wq,
                                 "quant_act": t_quant},
        "linear_tops": ops / ((t_quant + t_gemm) * 1e-3) / 1e12,
        "quant_act": {"GB/s": qbytes / (t_quant * 1e-3) / 1e9,
                      "frac_hbm": qbytes / (t_quant * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": qbytes},
        "per_tensor_act": {
            "act_absmax": _rate(ib * T * K + 4 * K, t_tabs),
            "quant_act_static": _rate(qbytes, t_qstat),
            "quant_act_per_tensor": _rate(qbytes + ib * T * K + 4 * K, t_qpt),
            "note": "bytes are algorithmic; the dynamic per-tensor quantiser reads X twice "
                    "(range, then codes)"},
        "norm_quant_act_rms": _rate(ib * T * K + 4 * K + T * K + 4 * T + 8 * T, t_norm),
        "fp8": {"quant_act": _rate(qbytes, t_q8), "gemm_us": t_g8 * 1e3,
                "gemm_TFLOP/s": ops / (t_g8 * 1e-3) / 1e12,
                "gemm_frac_fp8_peak": ops / (t_g8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                "linear_TFLOP/s": ops / ((t_q8 + t_g8) * 1e-3) / 1e12},
    }
    out.update(extra)
    if not args.no_cpu:
        del X, Xs, W, Wq, Xq, Y
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
