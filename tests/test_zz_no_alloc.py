"""rfx_gemv_noalloc (rfx_gemv with the library's own per-GPU scratch for
its split-K exchange slots) against rfx_gemv with a caller workspace, on
two calls in a row, the second with a smaller input: outputs bit-identical
(same kernels and launch shape) and within 1e-4 of the oracle."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
import oracle as O
from gpu_common import TOL, need_gpu, quantize_on_gpu, rel_err, say, upload_matrix, workspace

pytestmark = pytest.mark.gpu


def _case(torch, fmt, q, N, K, seed):
    W = inputgen.dense_weight(N, K, seed=seed, outliers=True)
    x = inputgen.activations(q, K, seed=seed + 1)
    dW = upload_matrix(torch, fmt, W)
    xq, xs, xsum = quantize_on_gpu(torch, x)
    return W, x, dW, xq, xs, xsum


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_gemv_noalloc_matches_gemv_with_workspace(fmt):
    torch = need_gpu()
    # both shapes split K across workgroups (the path that uses the scratch)
    for q, N, K, seed in ((4, 2048, 4096, 300 + fmt), (2, 200, 2080, 310 + fmt)):
        say(f"gemv noalloc fmt={fmt} q={q} N={N} K={K}")
        W, x, dW, xq, xs, xsum = _case(torch, fmt, q, N, K, seed)
        assert R.gemv_workspace_bytes(dW, q) > 0
        y_ws = torch.full((q, N), float("nan"), dtype=torch.float32, device="cuda")
        R.gemv(dW, xq, xs, xsum, q, y_ws, workspace(torch, R.gemv_workspace_bytes(dW, q)))
        y_na = torch.full((q, N), float("nan"), dtype=torch.float32, device="cuda")
        R.gemv_noalloc(dW, xq, xs, xsum, q, y_na)
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert np.array_equal(a, b)
        oq, os_ = O.quantize_act(x)
        yo = O.gemv(fmt, O.quantize_matrix(fmt, W), oq, os_)
        assert rel_err(b, yo) <= TOL


def test_gemv_noalloc_repeated_calls_leave_scratch_clear():
    """Many calls in a row on one stream: each must find its slots clear,
    so every result equals the first."""
    torch = need_gpu()
    W, x, dW, xq, xs, xsum = _case(torch, 3, 4, 1024, 2048, 320)
    outs = []
    for _ in range(5):
        y = torch.empty((4, 1024), dtype=torch.float32, device="cuda")
        R.gemv_noalloc(dW, xq, xs, xsum, 4, y)
        outs.append(y)
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy()
    for y in outs[1:]:
        assert np.array_equal(y.cpu().numpy(), first)
