"""GPU parity of the prefill-sized MoE layer (q > 4 tokens: fused router,
one-workgroup stable bucketing, grouped matrix-core gate/up + SwiGLU +
requantization, down, combine) against the oracle, stage by stage:

- the tokens' int8 activations bit-exact;
- routing bit-exact except at near-ties;
- bucketing = the oracle's stable bucketing of the GPU's indices, bit-exact;
- the GPU's fp32 h (the prefill test hook keeps it) within 1e-4 of the
  oracle's h, the GPU's h~ equal to the activation quantizer applied to the
  GPU's h (codes and scales bit-exact), and every code a valid rounding of
  the oracle's exact h within half a step plus 1e-4 (1 + |t|);
- the block dots the matrix core produced for probed work items (a routed
  expert's and the shared expert's; gate, up and down) equal to the
  oracle's exact integer dots;
- y within 1e-4 of the oracle fed the GPU's h~ (down, shared expert and
  combine).

The small layers are checked on every token and pair; the 2048-token
layer on every token's routing and on sampled experts, tokens and work
items (the oracle's FFN costs ~25 ms per (token, expert))."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
import oracle as O
from gpu_common import TOL, need_gpu, rel_err, say
from moe_common import LayerSpec, OracleMoe, check_routing

pytestmark = pytest.mark.gpu


def _items(spec, gpu, q):
    """The FFN work items the bucketing makes: (expert, first) per chunk of
    up to 64 tokens of one expert, then the shared expert's chunks."""
    counts = np.diff(gpu["expert_off"])
    out = [(e, f) for e in range(spec.n_experts) for f in range(0, int(counts[e]), 64)]
    if spec.shared:
        out += [(spec.n_experts, f) for f in range(0, q, 64)]
    return out


def _run(torch, spec, dev, x, k, resid=None, probes=None):
    """One prefill call, then the test hook: the fp32 h of every row and
    the block dots of each probed work item (default: the first and the
    last work item)."""
    q = x.shape[0]
    buf = R.MoeBuffers(dev, q, k)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    rd = None if resid is None else torch.from_numpy(np.ascontiguousarray(resid)).cuda()
    buf.run(dev, xd, resid=rd)
    torch.cuda.synchronize()
    out = {n: getattr(buf, n).cpu().numpy() for n in
           ("topk_idx", "topk_w", "pairs_sorted", "expert_off", "xq", "xs", "xsum", "y")}
    NP = q * k + q
    H, I = spec.hidden, spec.inter
    if probes is None:
        items = _items(spec, out, q)
        probes = sorted({items[0], items[-1]})
    h = torch.full((NP, I), float("nan"), dtype=torch.float32, device="cuda")
    out["dots"] = {}
    for i, (e, first) in enumerate(probes):
        dg = torch.full((I, 64, H // 32), -(2 ** 31), dtype=torch.int32, device="cuda")
        du = torch.full((I, 64, H // 32), -(2 ** 31), dtype=torch.int32, device="cuda")
        dd = torch.full((H, 64, I // 32), -(2 ** 31), dtype=torch.int32, device="cuda")
        R.moe_debug_prefill(dev, q, k, buf.xq, buf.xs, buf.topk_w, buf.pairs_sorted, buf.expert_off, buf.ws,
                            e, first, h=h if i == 0 else None, dots_gate=dg, dots_up=du, dots_down=dd)
        torch.cuda.synchronize()
        out["dots"][(e, first)] = (dg.cpu().numpy(), du.cpu().numpy(), dd.cpu().numpy())
        del dg, du, dd
    hq = torch.empty((NP, I), dtype=torch.int8, device="cuda")
    hs = torch.empty((NP, I // 32), dtype=torch.float32, device="cuda")
    R.moe_debug_hidden(dev, q, k, buf.ws, None, hq, hs)
    torch.cuda.synchronize()
    out.update(h=h.cpu().numpy(), hq=hq.cpu().numpy(), hs=hs.cpu().numpy())
    return out


def _check_front(spec, gpu, x, k, orc):
    """Activations, routing, bucketing. Returns the number of near-ties."""
    oq, os_ = O.quantize_act(x)
    assert np.array_equal(gpu["xq"], oq)
    assert np.array_equal(gpu["xs"].view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gpu["xsum"], O.act_sums(oq))
    ref = orc.route(x, k)
    near = check_routing(x, k, gpu, ref)
    idx = gpu["topk_idx"]
    # fp32 outputs: the 1e-4 bar (fp32 logits over 4096 terms carry ~1e-5)
    assert rel_err(gpu["topk_w"], np.take_along_axis(ref["probs"], idx.astype(np.int64), 1)) <= TOL
    ps, off = O.bucket(idx, spec.n_experts)
    assert np.array_equal(gpu["pairs_sorted"], ps) and np.array_equal(gpu["expert_off"], off)
    return near


def _check_hidden_rows(gpu, rows, h_ref):
    """GPU rows of h, h~ against the oracle's exact h of the same rows: h
    within 1e-4; h~ the quantizer of the GPU's own h, bit-exact; every code
    a valid rounding of the exact h (half a step plus 1e-4 (1 + |t|))."""
    rows = np.asarray(rows)
    h_g = gpu["h"][rows]
    for i in range(len(rows)):
        assert rel_err(h_g[i], h_ref[i]) <= TOL, rows[i]
    qq, ss = O.quantize_act(h_g)
    assert np.array_equal(gpu["hq"][rows], qq)
    assert np.array_equal(gpu["hs"][rows].view(np.uint32), ss.view(np.uint32))
    s = np.repeat(gpu["hs"][rows].astype(np.float64), 32, axis=1)
    t = np.divide(h_ref, s, out=np.zeros_like(h_ref), where=s > 0)
    assert np.all(np.abs(t - gpu["hq"][rows]) <= 0.5 + 1e-4 * (1 + np.abs(t)))


def _expert_h(orc, e, x_rows):
    oq, os_ = O.quantize_act(x_rows)
    return orc.expert_ffn(e, oq, os_)["h"]


def _item_rows(spec, gpu, q, k, e, first):
    """(h / o rows, tokens) of work item (e, first)."""
    if e == spec.n_experts:
        tok = np.arange(first, min(first + 64, q))
        return q * k + tok, tok
    off, ps = gpu["expert_off"], gpu["pairs_sorted"]
    pairs = ps[off[e] + first:min(off[e] + first + 64, off[e + 1])]
    return pairs, pairs // k


def _check_probe_dots(spec, orc, gpu, x, k, e, first):
    """Block dots of one work item, gate / up / down, against the oracle's
    exact integer dots on the same int8 inputs (down: the GPU's h~ rows)."""
    q = x.shape[0]
    rows, tok = _item_rows(spec, gpu, q, k, e, first)
    n = len(rows)
    dg, du, dd = gpu["dots"][(e, first)]
    oq, os_ = O.quantize_act(x[tok])
    for m, d in ((0, dg), (1, du)):
        fmt, blk = orc.blocks(e, m)
        _, do = O.gemv(fmt, blk, oq, os_, want_dots=True)       # [n][I][H/32]
        assert np.array_equal(d[:, :n, :].transpose(1, 0, 2), do), (e, first, m)
    fmt, blk = orc.blocks(e, 2)
    _, do = O.gemv(fmt, blk, gpu["hq"][rows], gpu["hs"][rows], want_dots=True)  # [n][H][I/32]
    assert np.array_equal(dd[:, :n, :].transpose(1, 0, 2), do), (e, first, "down")
    say(f"  block dots of item (expert {e}, first {first}, {n} tokens) bit-exact")


def _y_fed(spec, orc, gpu, x, k, t, resid=None):
    """Oracle y for token t with the GPU's h~ fed to every down projection."""
    q = x.shape[0]
    oq, os_ = O.quantize_act(x[t:t + 1])
    w = gpu["topk_w"][t].astype(np.float64)
    o_pairs = []
    for j in range(k):
        p = t * k + j
        e = int(gpu["topk_idx"][t][j])
        r = orc.expert_ffn(e, oq, os_, (gpu["hq"][p:p + 1], gpu["hs"][p:p + 1]))
        o_pairs.append(r["o"][0])
    if spec.shared:
        p = q * k + t
        o_sh = orc.expert_ffn(spec.n_experts, oq, os_, (gpu["hq"][p:p + 1], gpu["hs"][p:p + 1]))["o"]
    else:
        o_sh = np.zeros((1, spec.hidden))
    y = O.combine(o_sh, np.array(o_pairs)[None], w[None])[0]
    if resid is not None:
        y = y + resid[t].astype(np.float64)
    return y


def _check_all(spec, gpu, x, k, orc, resid=None):
    near = _check_front(spec, gpu, x, k, orc)
    q = x.shape[0]
    off, ps = gpu["expert_off"], gpu["pairs_sorted"]
    for e in range(spec.n_experts):
        pairs = ps[off[e]:off[e + 1]]
        if len(pairs) == 0:
            continue
        _check_hidden_rows(gpu, pairs, _expert_h(orc, e, x[pairs // k]))
    if spec.shared:
        _check_hidden_rows(gpu, np.arange(q * k, q * k + q), _expert_h(orc, spec.n_experts, x))
    for e, first in gpu["dots"]:
        _check_probe_dots(spec, orc, gpu, x, k, e, first)
    y_ref = np.array([_y_fed(spec, orc, gpu, x, k, t, resid) for t in range(q)])
    err = rel_err(gpu["y"], y_ref)
    say(f"  near-ties {near}, y err (fed h~) {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("q,k,shared,bias", [(5, 4, True, None), (37, 4, False, "zipf"), (130, 2, True, "zipf")])
def test_prefill_small(q, k, shared, bias):
    """Ragged token counts, experts with more than 64 tokens (several work
    items), with and without the shared expert and the Zipf bias."""
    torch = need_gpu()
    n_experts = 4 if q == 130 else 16
    say(f"prefill small q={q} k={k} E={n_experts} shared={shared} bias={bias}")
    spec = LayerSpec(layer=7, hidden=512, inter=288, n_experts=n_experts, shared=shared, bias=bias)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(7, q, q, spec.hidden)
    gpu = _run(torch, spec, dev, x, k)
    _check_all(spec, gpu, x, k, orc)


@pytest.mark.parametrize("fmts", [(4, 4, 2), (3, 2, 3)])
def test_prefill_other_formats(fmts):
    """Other format assignments (gate/up, down, shared) through the prefill
    kernels' codebook expansion: FP4 routed experts, FP2 / FP3 shared."""
    torch = need_gpu()
    fg, fd, fs = fmts
    say(f"prefill formats gate/up FP{fg} down FP{fd} shared FP{fs}")
    spec = LayerSpec(layer=11, hidden=512, inter=320, n_experts=8, shared=True,
                     fmt_gate=fg, fmt_down=fd, fmt_shared=fs)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(11, 0, 40, spec.hidden)
    gpu = _run(torch, spec, dev, x, 3)
    _check_all(spec, gpu, x, 3, orc)


def test_prefill_partial_tiles_and_residual():
    """hidden = 288 (gate/up K ends in a partial tile; the down output's last
    row group is half full), inter = 320, residual fused into the combine."""
    torch = need_gpu()
    spec = LayerSpec(layer=8, hidden=288, inter=320, n_experts=8, shared=True)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    q, k = 21, 3
    x = inputgen.tokens(8, 0, q, spec.hidden)
    resid = inputgen.tokens(8, 1, q, spec.hidden)
    gpu = _run(torch, spec, dev, x, k, resid)
    _check_all(spec, gpu, x, k, orc, resid)


def test_prefill_matches_decode_path_on_five_tokens():
    """Five tokens through the prefill path against the same tokens through
    the decode path in two calls (4 + 1): routing identical, y within 1e-4
    (the two paths sum the same blocks in the same order per output)."""
    torch = need_gpu()
    spec = LayerSpec(layer=9, hidden=1024, inter=512, n_experts=32, shared=True)
    dev = spec.build_device()
    x = inputgen.tokens(9, 0, 5, spec.hidden)
    pre = _run(torch, spec, dev, x, 6)
    idx, ys = [], []
    for sl in (slice(0, 4), slice(4, 5)):
        buf = R.MoeBuffers(dev, sl.stop - sl.start, 6)
        buf.run(dev, torch.from_numpy(np.ascontiguousarray(x[sl])).cuda())
        torch.cuda.synchronize()
        idx.append(buf.topk_idx.cpu().numpy())
        ys.append(buf.y.cpu().numpy())
    idx, ys = np.concatenate(idx), np.concatenate(ys)
    # the two routers sum the logits in different orders: a token whose
    # choice differs must be a near-tie for the oracle, and is not compared
    same = np.all(idx == pre["topk_idx"], axis=1)
    if not np.all(same):
        ref = O.route(x, spec.router_w, spec.router_b, 6)
        check_routing(x, 6, {"topk_idx": idx}, ref)
    assert same.sum() >= 4
    assert rel_err(pre["y"][same], ys[same]) <= TOL


def test_prefill_deterministic():
    torch = need_gpu()
    spec = LayerSpec(layer=10, hidden=512, inter=256, n_experts=16, shared=True)
    dev = spec.build_device()
    x = torch.from_numpy(inputgen.tokens(10, 0, 200, spec.hidden)).cuda()
    buf = R.MoeBuffers(dev, 200, 4)
    ys = []
    for _ in range(3):
        buf.run(dev, x)
        ys.append(buf.y.cpu().numpy().copy())
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_prefill_full_2048_tokens_top6():
    """The prefill-sized layer: 2048 tokens, hidden 4096, 256 experts,
    intermediate 2048, top-6, shared FP4 expert. Routing and bucketing on
    every token; h and h~ on eight sampled experts (every token they got)
    and on the shared expert for 64 tokens; the block dots of two work
    items (the busiest expert's first, the shared expert's at token 1024);
    y on 16 sampled tokens."""
    torch = need_gpu()
    say("prefill full: building 256 experts")
    spec = LayerSpec(layer=0, hidden=4096, inter=2048, n_experts=256, shared=True)
    dev = spec.build_device(workers=16)
    orc = OracleMoe(spec)
    q, k = 2048, 6
    x = inputgen.tokens(0, 1000, q, spec.hidden)
    # the bucketing is checked bit-exact against the oracle's below, so the
    # probed work items can be picked from the oracle's routing
    ref = orc.route(x, k)
    counts_ref = np.bincount(ref["idx"].reshape(-1), minlength=spec.n_experts)
    busiest = int(np.argmax(counts_ref))
    gpu = _run(torch, spec, dev, x, k, probes=[(busiest, 0), (spec.n_experts, 1024)])
    say("  checking routing")
    near = _check_front(spec, gpu, x, k, orc)
    off, ps = gpu["expert_off"], gpu["pairs_sorted"]
    counts = np.diff(off)
    say(f"  near-ties {near}; tokens per expert min {counts.min()} mean {counts.mean():.1f} max {counts.max()}")
    rng = np.random.default_rng(5)
    order = np.argsort(counts, kind="stable")
    sample_e = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2]), busiest}
                      | {int(e) for e in rng.choice(spec.n_experts, 5, replace=False)})
    sample_t = sorted(rng.choice(q, 16, replace=False).tolist())
    need = set(sample_e) | {int(e) for t in sample_t for e in gpu["topk_idx"][t]} | {spec.n_experts}
    orc.prefetch(sorted(need), workers=16)
    for e in sample_e:
        pairs = ps[off[e]:off[e + 1]]
        say(f"  expert {e}: {len(pairs)} tokens")
        _check_hidden_rows(gpu, pairs, _expert_h(orc, e, x[pairs // k]))
    tok = np.arange(1024, 1088)
    _check_hidden_rows(gpu, q * k + tok, _expert_h(orc, spec.n_experts, x[tok]))
    for e, first in gpu["dots"]:
        _check_probe_dots(spec, orc, gpu, x, k, e, first)
    y_ref = np.array([_y_fed(spec, orc, gpu, x, k, t) for t in sample_t])
    err = rel_err(gpu["y"][sample_t], y_ref)
    say(f"  y err on tokens {sample_t} (fed h~): {err:.2e}")
    assert err <= TOL


def test_prefill_uneven_expert_and_token_counts():
    """40 experts (the router's second 32-expert tile partial) and 77 tokens
    (the last 16-token tile partial), hidden 800 (no multiple of 256)."""
    torch = need_gpu()
    say("prefill uneven E=40 q=77")
    spec = LayerSpec(layer=13, hidden=800, inter=320, n_experts=40, shared=True)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(13, 77, 77, spec.hidden)
    gpu = _run(torch, spec, dev, x, 3)
    _check_all(spec, gpu, x, 3, orc)


def test_prefill_hidden_wider_than_the_h_rows():
    """hidden 1024 against inter 128 at top-1: the f16 copies of the token
    codes and of h~ that the FFN stages from take more than the fp32 h rows
    of the workspace region they live in (H > (k + 1) I), so the region must
    be sized for them; every stage is checked against the oracle."""
    torch = need_gpu()
    say("prefill hidden 1024 inter 128 k=1 q=96")
    spec = LayerSpec(layer=17, hidden=1024, inter=128, n_experts=8, shared=True)
    dev = spec.build_device()
    orc = OracleMoe(spec)
    x = inputgen.tokens(17, 96, 96, spec.hidden)
    gpu = _run(torch, spec, dev, x, 1)
    _check_all(spec, gpu, x, 1, orc)
