"""Shared helpers for the GPU parity tests (inputs, device upload, the
floored relative error the parity bar is stated in)."""

import sys

import numpy as np

import bit_block_quantized_amd as R


def need_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    R.lib()  # fail loudly if the HIP library is missing
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(y, ref):
    """max_n |y_n - ref_n| / max(|ref_n|, 0.01 * max|ref|): relative error
    with a floor so outputs near zero do not dominate."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = 0.01 * float(np.max(np.abs(ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), max(floor, 1e-300))
    return float(np.max(np.abs(y - ref) / den)) if ref.size else 0.0


TOL = 1e-4  # fp32 outputs against the fp64 oracle


def upload_matrix(torch, fmt, W):
    rows, cols = W.shape
    t = R.quantize_matrix(fmt, W)
    return R.DeviceQMat.from_host(fmt, rows, cols, t)


def quantize_on_gpu(torch, x):
    """Device fp32 [q][K] -> (xq, xs, xsum) device tensors via rfx_quantize_act."""
    q, K = x.shape
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    xq = torch.empty((q, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((q, K // 32), dtype=torch.float32, device="cuda")
    xsum = torch.empty((q, K // 32), dtype=torch.int32, device="cuda")
    R.quantize_act(xd, xq, xs, xsum)
    return xq, xs, xsum


def workspace(torch, nbytes):
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
