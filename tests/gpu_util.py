"""Helpers shared by the GPU parity tests (device transfer, bf16 views,
misaligned copies, the output tolerance check)."""
import numpy as np
import torch

import oracle as O

DEV = "cuda:0"


def dev_act(X, dtype):
    """float32 numpy array (bf16-representable when dtype is bf16) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(X, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        assert torch.equal(t.float(), torch.from_numpy(np.ascontiguousarray(X, np.float32)))
    return t.to(DEV)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_round(X):
    return torch.from_numpy(np.ascontiguousarray(X, np.float32)).to(torch.bfloat16).float().numpy()


def misaligned(t):
    """Same values in a contiguous tensor whose data pointer is 4 bytes off a
    16-byte boundary (forces the scalar kernels)."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    step = max(1, 4 // t.element_size())
    v = flat[step:step + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0 and v.is_contiguous()
    return v


def assert_out_close(y_gpu, y_ref32, out):
    """Contract tolerance against the oracle's fp32 output, plus equality with the
    oracle's own rounding (same epilogue order)."""
    if out == "f32":
        assert np.array_equal(y_gpu, y_ref32)
        assert np.all(np.abs(y_gpu - y_ref32) <= 1e-5 * np.abs(y_ref32))
    else:
        assert np.array_equal(y_gpu, O.to_bf16(y_ref32))
        yf = O.widen_bf16(y_gpu).astype(np.float64)
        r = y_ref32.astype(np.float64)
        assert np.all(np.abs(yf - r) <= 2.0 ** -8 * np.abs(r))
