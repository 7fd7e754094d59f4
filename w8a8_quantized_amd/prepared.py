"""Offline products of the layer, saved once and loaded by a serving process.

The smoothed, quantised weights belong to the checkpoint; nothing at inference
recomputes them (multigrid.ai "SmoothQuant Explained", section "Why the
rescaling is free at runtime").  A decomposition's outlier set, chosen once from
calibration, is stored the same way (mercemay.com "Activation Outlier Channels
and Mixed-Precision Decomposition", section "Decomposition: keep the outliers
in high precision").

The file is a NumPy .npz archive of plain arrays: loading uses
allow_pickle=False, so nothing in the file is executed.  Only the names below
are accepted, each with its dtype; sizes must agree (K input channels, N output
channels, n_o outlier channels).
"""
from __future__ import annotations

import numpy as np
import torch

# name -> (dtype, dimension names)
FIELDS = {
    "s": (np.float32, ("K",)),              # smoothing factors
    "x_absmax": (np.float32, ("K",)),       # calibration column maxima of X
    "w_absmax": (np.float32, ("K",)),       # column maxima of W
    "Wq": (np.int8, ("N", "K")),            # int8 weight codes of W diag(s)
    "Wq_fp8": (np.uint8, ("N", "K")),       # FP8 E4M3 weight codes of W diag(s)
    "w_scale": (np.float32, ("N",)),        # per-output-channel scales
    "outlier_idx": (np.int32, ("n_o",)),    # decomposition: outlier columns, ascending
    "outlier_mask": (np.float32, ("K",)),   # decomposition: 1 for kept columns, 0 for outliers
    "W_out": (np.float32, ("n_o", "N")),    # decomposition: outlier columns of W, outlier-major
    "alpha": (np.float64, ()),              # migration strength the factors were made with
}


def _check(arrays):
    dims = {}
    for name, a in arrays.items():
        if name not in FIELDS:
            raise ValueError(f"unknown field {name!r}")
        dt, shape = FIELDS[name]
        if a.dtype != dt:
            raise ValueError(f"{name}: dtype {a.dtype}, expected {np.dtype(dt)}")
        if a.ndim != len(shape):
            raise ValueError(f"{name}: {a.ndim} dimensions, expected {len(shape)}")
        for d, n in zip(shape, a.shape):
            if dims.setdefault(d, n) != n:
                raise ValueError(f"{name}: {d} = {n} disagrees with {dims[d]} from another field")
    return dims


def save_prepared(path, **tensors):
    """Write the given offline tensors (torch or NumPy; `alpha` a number) to an
    .npz file after checking names, dtypes and sizes."""
    arrays = {}
    for name, t in tensors.items():
        if t is None:
            continue
        if name == "alpha":
            arrays[name] = np.asarray(float(t), dtype=np.float64)
        elif isinstance(t, torch.Tensor):
            arrays[name] = t.detach().cpu().contiguous().numpy()
        else:
            arrays[name] = np.ascontiguousarray(t)
    _check(arrays)
    with open(path, "wb") as f:
        np.savez(f, **arrays)


def load_prepared(path, device="cuda"):
    """Read an archive written by save_prepared; returns a dict of torch tensors
    on `device` (and `alpha` as a float), after the same checks."""
    with np.load(path, allow_pickle=False) as z:
        arrays = {name: z[name] for name in z.files}
    _check(arrays)
    out = {}
    for name, a in arrays.items():
        out[name] = float(a) if name == "alpha" else torch.from_numpy(a.copy()).to(device)
    return out
