"""GPU tests of rfx_moe_forward, the whole MoE decode layer in one call: by
default the router launch computes the logits and every gate/up workgroup
picks the top k itself; with the one-launch flag, a single kernel for FP2
gate/up, FP3 down and an FP4 shared expert at q <= 4. Both compute the
two-call path's arithmetic (rfx_moe_route_topk + rfx_moe_ffn) step for
step, so every output is compared with that path bit for bit, and the layer
is also checked stage by stage against the oracle. The one-launch kernel's
counters must return to zero after every call: repeated calls on the same
buffers, graph replays and the chained eight-layer stack check that, and
the time-bound status word must stay clear."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
from gpu_common import need_gpu, say
from moe_common import LayerSpec, OracleMoe
from test_gpu_moe import _check_layer

pytestmark = pytest.mark.gpu

OUTS = ("topk_idx", "topk_w", "pairs_sorted", "expert_off", "xq", "xs", "xsum", "y")


def _hidden(torch, dev, buf):
    q, k = buf.q, buf.k
    NP = q * k + q
    h = torch.empty((NP, dev.inter), dtype=torch.float32, device="cuda")
    hq = torch.empty((NP, dev.inter), dtype=torch.int8, device="cuda")
    hs = torch.empty((NP, dev.inter // 32), dtype=torch.float32, device="cuda")
    R.moe_debug_hidden(dev, q, k, buf.ws, h, hq, hs)
    torch.cuda.synchronize()
    return h.cpu().numpy(), hq.cpu().numpy(), hs.cpu().numpy()


def _read(torch, dev, buf):
    torch.cuda.synchronize()
    out = {n: getattr(buf, n).cpu().numpy() for n in OUTS}
    out["h"], out["hq"], out["hs"] = _hidden(torch, dev, buf)
    return out


def _same(a, b, what):
    """Bit-identical arrays (fp32 compared as bit patterns)."""
    for n in a:
        x, y = np.asarray(a[n]), np.asarray(b[n])
        if x.dtype == np.float32:
            x, y = x.view(np.uint32), y.view(np.uint32)
        assert x.shape == y.shape and np.array_equal(x, y), f"{what}: {n} differs"


def _both(torch, dev, x, k, resid=False, single=True):
    """The layer through moe_forward (one-launch flag) and through the two
    calls, on separate buffers, for the same tokens; the default forward
    path (routing inside the gate/up workgroups) must equal the two calls
    too. Returns (one-launch forward outputs, two-call outputs, buffers)."""
    q = x.shape[0]
    assert R.moe_forward_single_launch(dev, q, k) == single
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf, br, b0 = R.MoeBuffers(dev, q, k), R.MoeBuffers(dev, q, k), R.MoeBuffers(dev, q, k)
    bf.forward(dev, xd, resid=xd if resid else None, one_launch=True)
    br.run(dev, xd, resid=xd if resid else None)
    b0.forward(dev, xd, resid=xd if resid else None)
    f, r = _read(torch, dev, bf), _read(torch, dev, br)
    _same(_read(torch, dev, b0), r, "routed forward vs two calls")
    R.moe_forward_status(dev, q, k, bf.ws)
    return f, r, bf


@pytest.mark.parametrize("q", [1, 2, 3, 4])
@pytest.mark.parametrize("shared,bias", [(True, None), (False, "zipf"), (True, "zipf")])
def test_forward_small_matches_two_calls_and_oracle(q, shared, bias):
    """Ragged sizes (intermediate 288: a partial row group and a partial
    tile), 16 experts, top-4."""
    torch = need_gpu()
    say(f"moe forward small q={q} shared={shared} bias={bias}")
    spec = LayerSpec(layer=3, hidden=512, inter=288, n_experts=16, shared=shared, bias=bias)
    dev = spec.build_device()
    x = inputgen.tokens(3, q, q, spec.hidden)
    f, r, _ = _both(torch, dev, x, 4)
    _same(f, r, "forward vs two calls")
    _check_layer(spec, f, x, 4, OracleMoe(spec))


def test_forward_k_edges_and_shared_picks():
    """k = 1 and k = 8, tokens that pick the same experts (one expert
    decoded for several tokens), more pairs than experts, and the residual
    fused into the combine."""
    torch = need_gpu()
    spec = LayerSpec(layer=5, hidden=256, inter=256, n_experts=8, shared=True)
    spec.router_b = np.array([9, 8, 0, 0, 0, 0, 7, 0], np.float32)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    for q, k in ((4, 3), (4, 1), (2, 8), (3, 6), (4, 8)):
        say(f"moe forward edges q={q} k={k}")
        x = inputgen.tokens(5, 10 + q + k, q, spec.hidden)
        f, r, _ = _both(torch, dev, x, k, resid=True)
        _same(f, r, f"q={q} k={k}")
        _check_layer(spec, f, x, k, orc, resid=x)


@pytest.mark.parametrize("q,k", [(1, 1), (2, 4), (4, 8)])
def test_forward_default_routes_in_gateup(q, k):
    """Without the one-launch flag the gate/up workgroups pick the top k
    from the router's logits; every routing output (written by one
    workgroup) and y equal the two calls'. Small workgroups (few slots, one
    wave per workgroup for some shapes) and all k."""
    torch = need_gpu()
    spec = LayerSpec(layer=4, hidden=512, inter=256, n_experts=16, shared=True, bias="zipf")
    dev = spec.build_device()
    x = inputgen.tokens(4, q + 10 * k, q, spec.hidden)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bf, br = R.MoeBuffers(dev, q, k), R.MoeBuffers(dev, q, k)
    bf.forward(dev, xd, resid=xd)
    br.run(dev, xd, resid=xd)
    _same(_read(torch, dev, bf), _read(torch, dev, br), f"flags = 0, q={q} k={k}")


@pytest.mark.parametrize("fmts", [(4, 4, 2), (3, 2, 3)])
def test_forward_other_formats_take_two_calls(fmts):
    """Format assignments the one-launch kernel is not built for go through
    the two calls, with the same results."""
    torch = need_gpu()
    fg, fd, fs = fmts
    spec = LayerSpec(layer=7, hidden=512, inter=320, n_experts=8, shared=True, fmt_gate=fg, fmt_down=fd,
                     fmt_shared=fs)
    dev = spec.build_device()
    x = inputgen.tokens(7, 30, 2, spec.hidden)
    f, r, _ = _both(torch, dev, x, 3, single=False)
    _same(f, r, "fallback")


@pytest.mark.parametrize("one_launch", [True, False])
def test_forward_repeated_calls_reset_counters(one_launch):
    """Consecutive calls on the same buffers with different tokens and
    token counts' worth of routing: each call's outputs equal the two-call
    path's for the same tokens (a counter left non-zero by one call would
    release the next call's waits early)."""
    torch = need_gpu()
    spec = LayerSpec(layer=6, hidden=1024, inter=512, n_experts=32, shared=True, bias="zipf")
    dev = spec.build_device()
    for q in (1, 4):
        bf, br = R.MoeBuffers(dev, q, 4), R.MoeBuffers(dev, q, 4)
        for i in range(6):
            xd = torch.from_numpy(inputgen.tokens(6, 100 + i, q, spec.hidden)).cuda()
            bf.forward(dev, xd, resid=xd, one_launch=one_launch)
            br.run(dev, xd, resid=xd)
            _same(_read(torch, dev, bf), _read(torch, dev, br), f"q={q} call {i}")
        R.moe_forward_status(dev, q, 4, bf.ws)
        sync = bf.ws.cpu().numpy()
        say(f"  q={q}: workspace words non-zero after the calls: {int(np.count_nonzero(sync))}")


@pytest.mark.parametrize("one_launch", [True, False])
def test_forward_graph_replays(one_launch):
    """Three layers' forward calls captured in one graph and replayed four
    times with eager work in between; every replay's outputs equal the
    eager results."""
    torch = need_gpu()
    specs = [LayerSpec(layer=l, hidden=512, inter=256, n_experts=64, shared=True, bias="zipf") for l in range(3)]
    devs = [s.build_device() for s in specs]
    q, k = 2, 4
    bufs = [R.MoeBuffers(d, q, k) for d in devs]
    xs = [torch.from_numpy(inputgen.tokens(40, 0, q, 512)).cuda()]
    xs += [torch.empty((q, 512), dtype=torch.float32, device="cuda") for _ in devs]

    def chain():
        for l, d in enumerate(devs):
            bufs[l].forward(d, xs[l], resid=xs[l], out=xs[l + 1], one_launch=one_launch)

    chain()
    torch.cuda.synchronize()
    ref = [_read(torch, d, b) for d, b in zip(devs, bufs)]
    ref_x = [t.cpu().numpy() for t in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for rep in range(4):
        for t in xs[1:]:  # the chain's outputs (out=), cleared before each replay
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, (d, b) in enumerate(zip(devs, bufs)):
            _same(_read(torch, d, b), ref[l], f"replay {rep} layer {l}")
            assert np.array_equal(xs[l + 1].cpu().numpy().view(np.uint32), ref_x[l + 1].view(np.uint32))
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between replays
    for d, b in zip(devs, bufs):
        R.moe_forward_status(d, q, k, b.ws)


def _stack(torch, devs, x0, k, fused, one_launch=True):
    q, H = x0.shape[0], devs[0].hidden
    bufs = [R.MoeBuffers(d, q, k) for d in devs]
    xb = [torch.from_numpy(np.ascontiguousarray(x0)).cuda()]
    xb += [torch.empty((q, H), dtype=torch.float32, device="cuda") for _ in devs]
    for l, d in enumerate(devs):
        if fused:
            bufs[l].forward(d, xb[l], resid=xb[l], out=xb[l + 1], one_launch=one_launch)
        else:
            bufs[l].run(d, xb[l], resid=xb[l], out=xb[l + 1])
    torch.cuda.synchronize()
    outs = []
    for l, (d, b) in enumerate(zip(devs, bufs)):
        o = _read(torch, d, b)
        o.pop("y")
        o["x"], o["y"] = xb[l].cpu().numpy(), xb[l + 1].cpu().numpy()
        outs.append(o)
    if fused:
        for d, b in zip(devs, bufs):
            R.moe_forward_status(d, q, k, b.ws)
    return outs


@pytest.mark.parametrize("q", [1, 4])
def test_forward_stack_eight_layers(q):
    """The stacked workload as benchmarked with the one-launch layer: eight
    layers chained on the device with the residual fused (top-4, Zipf(1.1)
    bias, shared FP4 expert) at a reduced size; equal to the two-call
    chain, and each layer checked with the oracle fed the GPU's x_l."""
    torch = need_gpu()
    say(f"moe forward stack 8 q={q}")
    specs = [LayerSpec(layer=l, hidden=512, inter=256, n_experts=64, shared=True, bias="zipf") for l in range(8)]
    devs = [s.build_device() for s in specs]
    x0 = inputgen.tokens(100, 0, q, 512)
    fo = _stack(torch, devs, x0, 4, True)
    ro = _stack(torch, devs, x0, 4, False)
    f0 = _stack(torch, devs, x0, 4, True, one_launch=False)
    for l in range(8):
        _same(fo[l], ro[l], f"layer {l}")
        _same(f0[l], ro[l], f"routed forward, layer {l}")
    for l, (spec, gpu) in enumerate(zip(specs, fo)):
        _check_layer(spec, gpu, gpu["x"], 4, OracleMoe(spec), resid=gpu["x"])


@pytest.mark.parametrize("q,k,bias", [(1, 4, "zipf"), (4, 6, None)])
def test_forward_full_size(q, k, bias):
    """Full size (256 experts, hidden 4096, intermediate 2048, FP2 gate/up,
    FP3 down, FP4 shared): q = 1 top-4 with the Zipf bias (the stacked
    workload's first layer and tokens) and q = 4 top-6; equal to the two
    calls, and checked against the oracle."""
    torch = need_gpu()
    say(f"moe forward full size q={q} k={k}: building 256 experts")
    spec = LayerSpec(layer=0, hidden=4096, inter=2048, n_experts=256, shared=True, bias=bias)
    dev = spec.build_device(workers=16)
    x = inputgen.tokens(100, 0, q, 4096) if bias else inputgen.tokens(0, 0, q, 4096)
    f, r, _ = _both(torch, dev, x, k, resid=bias is not None)
    _same(f, r, "full size")
    orc = OracleMoe(spec)
    orc.prefetch(sorted(set(f["topk_idx"].reshape(-1).tolist())) + [spec.n_experts], workers=16)
    _check_layer(spec, f, x, k, orc, resid=x if bias else None)
    del dev
    torch.cuda.empty_cache()
