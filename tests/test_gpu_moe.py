"""GPU parity of the MoE decode layer (router, fused gate/up + SwiGLU +
requantization, down + shared expert + combine) against the oracle, in
stages: routing bit-exact (near-ties excepted), h within 1e-4, h~ equal to
the quantizer of the GPU's h, down + combine within 1e-4 given the GPU's h~,
and the free-running end-to-end error reported (it differs from the fed
result only where an h element sits on a rounding midpoint within fp32
noise, which is checked element by element)."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
import oracle as O
from gpu_common import TOL, need_gpu, rel_err, say
from moe_common import LayerSpec, OracleMoe, check_routing

pytestmark = pytest.mark.gpu


def _run_layer(torch, spec, dev, x, k):
    q = x.shape[0]
    buf = R.MoeBuffers(dev, q, k)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    buf.run(dev, xd)
    NP = q * k + q
    h = torch.empty((NP, spec.inter), dtype=torch.float32, device="cuda")
    hq = torch.empty((NP, spec.inter), dtype=torch.int8, device="cuda")
    hs = torch.empty((NP, spec.inter // 32), dtype=torch.float32, device="cuda")
    R.moe_debug_hidden(dev, q, k, buf.ws, h, hq, hs)
    torch.cuda.synchronize()
    out = {n: getattr(buf, n).cpu().numpy() for n in
           ("topk_idx", "topk_w", "pairs_sorted", "expert_off", "xq", "xs", "xsum", "y")}
    out.update(h=h.cpu().numpy(), hq=hq.cpu().numpy(), hs=hs.cpu().numpy(), buf=buf)
    return out


def _check_layer(spec, gpu, x, k, orc, resid=None):
    """Stage-wise parity of one layer. With resid (the layer's input, as
    the stacked workload fuses x_{l+1} = x_l + y_l), the GPU output is the
    sum and every reference y has resid added in fp64."""
    q = x.shape[0]
    # activations of the tokens: bit-exact
    oq, os_ = O.quantize_act(x)
    assert np.array_equal(gpu["xq"], oq)
    assert np.array_equal(gpu["xs"].view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gpu["xsum"], O.act_sums(oq))
    # routing
    ref = orc.route(x, k)
    near = check_routing(x, k, gpu, ref)
    idx = gpu["topk_idx"]
    assert rel_err(gpu["topk_w"], np.take_along_axis(ref["probs"], idx.astype(np.int64), 1)) <= 1e-5
    ps, off = O.bucket(idx, spec.n_experts)
    assert np.array_equal(gpu["pairs_sorted"], ps) and np.array_equal(gpu["expert_off"], off)
    # h and its requantization, with the GPU's routing
    w = gpu["topk_w"].astype(np.float64)
    y_own, h_ref, hq_ref, hs_ref = orc.layer(x, k, idx, w)
    NP = q * k + q
    rows = range(q * k) if not spec.shared else range(NP)
    for p in rows:
        assert rel_err(gpu["h"][p], h_ref[p]) <= TOL, p
        qq, ss = O.quantize_act(gpu["h"][p])
        assert np.array_equal(gpu["hq"][p], qq), p
        assert np.array_equal(gpu["hs"][p].view(np.uint32), ss.view(np.uint32)), p
    # every GPU code is a valid rounding of the oracle's exact h: within
    # half a step plus fp32 noise (a "flip" is a rounding-midpoint case)
    rr = list(rows)
    s_g = np.repeat(gpu["hs"][rr].astype(np.float64), 32, axis=1)
    t = np.divide(h_ref[rr], s_g, out=np.zeros_like(h_ref[rr]), where=s_g > 0)
    assert np.all(np.abs(t - gpu["hq"][rr]) <= 0.5 + 1e-4 * (1 + np.abs(t)))
    # down + shared + combine given the GPU's h~
    y_fed, _, _, _ = orc.layer(x, k, idx, w, gpu["hq"], gpu["hs"])
    r64 = np.zeros_like(y_fed) if resid is None else np.asarray(resid, np.float64)
    y_gpu = gpu["y"].astype(np.float64)
    err = rel_err(y_gpu, y_fed + r64)
    assert err <= TOL
    # Free-running: the oracle's own h~ instead of the GPU's. The two runs
    # differ only where h~ differs (a flip at a rounding midpoint, or a
    # block scale one fp32 ulp apart), so |y_gpu - y_own| is at most the
    # fed error plus the requantization bound of those differences; with
    # no difference the fed bar applies as is.
    hq_g = np.zeros_like(hq_ref)
    hs_g = np.zeros_like(hs_ref)
    hq_g[rr], hs_g[rr] = gpu["hq"][rr], gpu["hs"][rr]
    bound, n_diff = orc.requant_bound(q, k, idx, w, hq_g, hs_g, hq_ref, hs_ref)
    flips = int(np.sum(gpu["hq"][rr] != hq_ref[rr]))
    free = rel_err(y_gpu, y_own + r64)
    d_free = np.abs(y_gpu - (y_own + r64))
    d_fed = np.abs(y_gpu - (y_fed + r64))
    floor = 0.01 * float(np.max(np.abs(y_own + r64)))
    bound_rel = float(np.max(bound / np.maximum(np.abs(y_own + r64), floor)))
    say(f"  near-ties {near}, y err (fed h~) {err:.2e}, h~ flips {flips} ({n_diff} elements differ), "
        f"free-running err {free:.2e}, requant bound {bound_rel:.2e}")
    assert np.all(d_free <= d_fed + bound + 1e-9 * (1.0 + np.abs(y_own + r64)))
    if n_diff == 0:
        assert free <= TOL
    return {"near": near, "err": err, "flips": flips, "free": free, "bound": bound_rel}


@pytest.mark.parametrize("q", [1, 2, 3, 4])
@pytest.mark.parametrize("shared,bias", [(True, None), (False, "zipf"), (True, "zipf")])
def test_moe_small(q, shared, bias):
    torch = need_gpu()
    say(f"moe small q={q} shared={shared} bias={bias}")
    spec = LayerSpec(layer=3, hidden=512, inter=288, n_experts=16, shared=shared, bias=bias)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(3, q, q, spec.hidden)
    gpu = _run_layer(torch, spec, dev, x, k=4)
    _check_layer(spec, gpu, x, 4, orc)


@pytest.mark.parametrize("fmts", [(4, 4, 2), (3, 2, 3), (4, 3, 4)])
@pytest.mark.parametrize("q", [1, 2, 4])
def test_moe_other_formats(fmts, q):
    """Other format assignments (gate/up, down, shared): FP4 routed experts
    (their one- and two-token slots take the block-scaled matrix core for
    gate/up and down), FP2 / FP3 shared experts (the vector paths for the
    shared slot), with experts picked by several tokens."""
    torch = need_gpu()
    fg, fd, fs = fmts
    say(f"moe formats gate/up FP{fg} down FP{fd} shared FP{fs} q={q}")
    spec = LayerSpec(layer=7, hidden=512, inter=320, n_experts=8, shared=True,
                     fmt_gate=fg, fmt_down=fd, fmt_shared=fs)
    spec.router_b = np.array([6, 0, 5, 0, 0, 0, 0, 0], np.float32)  # experts 0, 2 for most tokens
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(7, 20 + q, q, spec.hidden)
    gpu = _run_layer(torch, spec, dev, x, k=3)
    _check_layer(spec, gpu, x, 3, orc)


def test_moe_shared_token_experts_and_k_edges():
    """Tokens that pick the same experts (one expert decoded for several
    tokens), k = 1 and k = 8, and more pairs than experts."""
    torch = need_gpu()
    spec = LayerSpec(layer=5, hidden=256, inter=256, n_experts=8, shared=True)
    spec.router_b = np.array([9, 8, 0, 0, 0, 0, 7, 0], np.float32)  # 0, 1, 6 for everyone
    dev = spec.build_device()
    orc = OracleMoe(spec)
    for q, k in ((4, 3), (4, 1), (2, 8), (3, 6)):
        say(f"moe edges q={q} k={k}")
        x = inputgen.tokens(5, 10 + q + k, q, spec.hidden)
        gpu = _run_layer(torch, spec, dev, x, k)
        _check_layer(spec, gpu, x, k, orc)


def test_moe_deterministic():
    torch = need_gpu()
    spec = LayerSpec(layer=6, hidden=1024, inter=512, n_experts=32, shared=True)
    dev = spec.build_device()
    x = torch.from_numpy(inputgen.tokens(6, 0, 4, spec.hidden)).cuda()
    buf = R.MoeBuffers(dev, 4, 6)
    ys = []
    for _ in range(3):
        buf.run(dev, x)
        ys.append(buf.y.cpu().numpy().copy())
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_moe_layer_full_size_q4_top6():
    """One MoE decode layer at full size: 256 experts, hidden 4096,
    intermediate 2048, FP2 gate/up, FP3 down, FP4 shared, top-6, q = 4."""
    torch = need_gpu()
    say("moe full layer: building 256 experts")
    spec = LayerSpec(layer=0, hidden=4096, inter=2048, n_experts=256, shared=True)
    dev = spec.build_device(workers=16)
    orc = OracleMoe(spec)
    x = inputgen.tokens(0, 0, 4, spec.hidden)
    gpu = _run_layer(torch, spec, dev, x, k=6)
    used = sorted(set(gpu["topk_idx"].reshape(-1).tolist()))
    say(f"  distinct experts {len(used)}")
    orc.prefetch(used + [spec.n_experts], workers=16)
    _check_layer(spec, gpu, x, 6, orc)


def _stack_chain(torch, devs, x0, k):
    """The stacked workload as the benchmark runs it: each layer's call
    reads x_l and writes x_{l+1} = x_l + MoE(x_l) (the residual fused into
    the combine), layer after layer on the device, each layer with its own
    buffers. Returns per-layer output dicts (x_l, routing, h, h~, y =
    x_{l+1}) read back after the whole chain ran."""
    q = x0.shape[0]
    H = devs[0].hidden
    bufs = [R.MoeBuffers(dev, q, k) for dev in devs]
    xbuf = [torch.from_numpy(np.ascontiguousarray(x0)).cuda()]
    xbuf += [torch.empty((q, H), dtype=torch.float32, device="cuda") for _ in devs]
    for l, dev in enumerate(devs):
        bufs[l].run(dev, xbuf[l], resid=xbuf[l], out=xbuf[l + 1])
    torch.cuda.synchronize()
    outs = []
    NP = q * k + q
    for l, (dev, buf) in enumerate(zip(devs, bufs)):
        h = torch.empty((NP, dev.inter), dtype=torch.float32, device="cuda")
        hq = torch.empty((NP, dev.inter), dtype=torch.int8, device="cuda")
        hs = torch.empty((NP, dev.inter // 32), dtype=torch.float32, device="cuda")
        R.moe_debug_hidden(dev, q, k, buf.ws, h, hq, hs)
        torch.cuda.synchronize()
        o = {n: getattr(buf, n).cpu().numpy() for n in
             ("topk_idx", "topk_w", "pairs_sorted", "expert_off", "xq", "xs", "xsum")}
        o.update(h=h.cpu().numpy(), hq=hq.cpu().numpy(), hs=hs.cpu().numpy(),
                 x=xbuf[l].cpu().numpy(), y=xbuf[l + 1].cpu().numpy())
        outs.append(o)
    return outs


@pytest.mark.parametrize("q", [1, 4])
def test_moe_stack_eight_layers_fused_residual(q):
    """All eight layers of the stacked workload chained on the device with
    the residual fused, as benchmarked (top-4, Zipf(1.1) router bias, shared
    FP4 expert), at a reduced size (hidden 512, intermediate 256, 64
    experts); each layer checked with the oracle fed the GPU's x_l, the
    residual included in y."""
    torch = need_gpu()
    say(f"moe stack 8 layers fused residual q={q}")
    specs = [LayerSpec(layer=l, hidden=512, inter=256, n_experts=64, shared=True, bias="zipf") for l in range(8)]
    devs = [s.build_device() for s in specs]
    outs = _stack_chain(torch, devs, inputgen.tokens(100, 0, q, 512), k=4)
    for l, (spec, gpu) in enumerate(zip(specs, outs)):
        say(f" layer {l}")
        _check_layer(spec, gpu, gpu["x"], 4, OracleMoe(spec), resid=gpu["x"])


@pytest.mark.parametrize("q", [1, 4])
def test_moe_stack_full_size_fused_residual(q):
    """The first two layers of the stacked workload at full size (256
    experts, hidden 4096, intermediate 2048, top-4, Zipf(1.1) bias, the
    benchmark's layer seeds and first tokens), chained on the device with
    the residual fused exactly as benchmarked; each layer checked with the
    oracle fed the GPU's x_l."""
    torch = need_gpu()
    specs, devs = [], []
    for layer in (0, 1):
        say(f"moe stack full size q={q}: building layer {layer}")
        specs.append(LayerSpec(layer=layer, hidden=4096, inter=2048, n_experts=256, shared=True, bias="zipf"))
        devs.append(specs[-1].build_device(workers=16))
    outs = _stack_chain(torch, devs, inputgen.tokens(100, 0, q, 4096), k=4)
    for l, (spec, gpu) in enumerate(zip(specs, outs)):
        orc = OracleMoe(spec)
        orc.prefetch(sorted(set(gpu["topk_idx"].reshape(-1).tolist())) + [spec.n_experts], workers=16)
        say(f" layer {l}")
        _check_layer(spec, gpu, gpu["x"], 4, orc, resid=gpu["x"])
    del devs
    torch.cuda.empty_cache()


def test_moe_router_exact_ties_go_to_lower_id():
    """Experts with identical router rows and biases have bit-identical
    logits on both sides, so the tie rule (equal logits to the lower id)
    decides their order. The tied groups sit in one lane of the router's
    wave (experts 5, 69, 133, 197 share a lane), across lanes (10, 11,
    12, 74) and at the ends of the id range (0, 255); k = 6 splits a
    group."""
    torch = need_gpu()
    spec = LayerSpec(layer=9, hidden=256, inter=64, n_experts=256, shared=False)
    groups = ([5, 69, 133, 197], [74, 12, 10, 11], [255, 0])
    w = spec.router_w.copy()
    b = np.zeros(spec.n_experts, np.float32)
    for gi, g in enumerate(groups):
        for e in g:
            w[e] = w[g[0]]
            b[e] = 8.0 - gi
    spec.router_w, spec.router_b = w, b
    dev = spec.build_device()
    orc = OracleMoe(spec)
    for q, k in ((4, 8), (4, 6), (1, 3), (3, 2)):
        say(f"router ties q={q} k={k}")
        x = inputgen.tokens(9, 40 + q + k, q, spec.hidden)
        ref = orc.route(x, k)
        # the groups' logits are far apart for these tokens, so only the
        # exact ties inside a group decide the order
        for t in range(q):
            lg = sorted(ref["logits"][t][g[0]] for g in groups)
            assert min(np.diff(lg)) > 1e-3
        gpu = _run_layer(torch, spec, dev, x, k)
        assert np.array_equal(gpu["topk_idx"], ref["idx"]), (gpu["topk_idx"], ref["idx"])
        _check_layer(spec, gpu, x, k, orc)


@pytest.mark.parametrize("n_experts", [200, 100])
@pytest.mark.parametrize("q", [1, 4])
def test_moe_uneven_expert_count_and_hidden(n_experts, q):
    """Expert counts that leave the router's last arrival group partial
    (200: 13 groups of 16, the last of 8) and the last candidate row of
    its top-k wave partly empty, with a hidden size that is no multiple of
    the 256-column tile (800) and top-6."""
    torch = need_gpu()
    say(f"moe uneven E={n_experts} q={q}")
    spec = LayerSpec(layer=12, hidden=800, inter=320, n_experts=n_experts, shared=True)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(12, n_experts + q, q, spec.hidden)
    gpu = _run_layer(torch, spec, dev, x, k=6)
    _check_layer(spec, gpu, x, 6, orc)
