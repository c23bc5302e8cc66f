"""Expert placement: routed experts split between device memory (hot) and
pinned host memory (cold), reached through the layer's per-expert pointer
table. The kernels read the same bytes wherever they sit, so the results
must equal those of the stacked layout bit for bit (decode at q = 1..4,
prefill), and stay within the oracle's bar."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
from gpu_common import need_gpu, say
from moe_common import LayerSpec, OracleMoe
from test_gpu_moe import _check_layer, _run_layer

pytestmark = pytest.mark.gpu


def _y(torch, layer, x, k, resid=None):
    q = x.shape[0]
    buf = R.MoeBuffers(layer, q, k)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    rd = None if resid is None else torch.from_numpy(np.ascontiguousarray(resid)).cuda()
    buf.run(layer, xd, resid=rd)
    torch.cuda.synchronize()
    return buf.y.cpu().numpy(), buf.topk_idx.cpu().numpy()


def test_placed_layer_equals_stacked_layer():
    torch = need_gpu()
    spec = LayerSpec(layer=21, hidden=512, inter=256, n_experts=16, shared=True, bias="zipf")
    dev = spec.build_device()
    counts = np.exp(spec.router_b.astype(np.float64))  # the bias ranks the experts
    hot = R.layer.hot_experts_by_frequency(counts, 6)
    placed = R.PlacedMoeLayer(dev, hot)
    assert placed.hot == hot and len(placed.cold) == 10
    cold_hits = 0
    for q, k in ((1, 4), (2, 4), (3, 6), (4, 6), (37, 4)):
        say(f"placement q={q} k={k}")
        x = inputgen.tokens(21, q, q, spec.hidden)
        resid = inputgen.tokens(21, 100 + q, q, spec.hidden)
        y0, idx0 = _y(torch, dev, x, k, resid)
        y1, idx1 = _y(torch, placed, x, k, resid)
        assert np.array_equal(idx0, idx1)
        assert np.array_equal(y0, y1)
        cold_hits += int(np.isin(idx1, placed.cold).sum())
    assert cold_hits > 0  # some picks read host memory
    # the placed layer against the oracle, stage by stage
    x = inputgen.tokens(21, 50, 4, spec.hidden)
    gpu = _run_layer(torch, spec, placed, x, 6)
    _check_layer(spec, gpu, x, 6, OracleMoe(spec))


def test_placed_full_size_layer_equals_stacked_layer():
    """256 experts at full size, 64 in HBM and 192 in host memory, q = 1
    and 4 decode."""
    torch = need_gpu()
    say("placement full size: building 256 experts")
    spec = LayerSpec(layer=3, hidden=4096, inter=2048, n_experts=256, shared=True, bias="zipf")
    dev = spec.build_device(workers=16)
    hot = R.layer.hot_experts_by_frequency(np.exp(spec.router_b.astype(np.float64)), 64)
    placed = R.PlacedMoeLayer(dev, hot)
    hb, cb = placed.hbm_bytes()
    say(f"  routed experts: {hb / 2**30:.2f} GiB in HBM, {cb / 2**30:.2f} GiB in host memory")
    for q, k in ((1, 4), (4, 4)):
        x = inputgen.tokens(3, q, q, spec.hidden)
        y0, idx0 = _y(torch, dev, x, k)
        y1, idx1 = _y(torch, placed, x, k)
        assert np.array_equal(idx0, idx1) and np.array_equal(y0, y1)
        say(f"  q={q}: {int(np.isin(idx1, placed.cold).sum())} of {idx1.size} picks in host memory, y equal")
    del placed, dev
    torch.cuda.empty_cache()
