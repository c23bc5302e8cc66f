"""MoE test helpers: a seeded layer description shared by the GPU build and
the oracle, the oracle side (encodes only the experts a test touches), and
the stage-wise comparison."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import inputgen
import oracle as O
from gpu_common import rel_err


class LayerSpec:
    def __init__(self, layer, hidden, inter, n_experts, shared=True, bias=None,
                 fmt_gate=2, fmt_down=3, fmt_shared=4):
        self.layer, self.hidden, self.inter, self.n_experts = layer, hidden, inter, n_experts
        self.shared, self.fmt_gate, self.fmt_down, self.fmt_shared = shared, fmt_gate, fmt_down, fmt_shared
        self.router_w = inputgen.router_weight(layer, n_experts, hidden)
        if bias == "zipf":
            self.router_b = inputgen.zipf_router_bias(layer, n_experts)
        else:
            self.router_b = bias

    def weight(self, e, mat, rows, cols):
        return inputgen.expert_weight(self.layer, e, mat, rows, cols)

    def build_device(self, workers=8):
        import bit_block_quantized_amd as R
        return R.DeviceMoeLayer.build(self.hidden, self.inter, self.n_experts, self.weight,
                                      self.router_w, self.router_b, fmt_gate=self.fmt_gate,
                                      fmt_down=self.fmt_down, fmt_shared=self.fmt_shared,
                                      shared=self.shared, workers=workers)


class OracleMoe:
    """The oracle's view of a layer: blocks encoded by the oracle itself."""

    def __init__(self, spec: LayerSpec):
        self.s = spec
        self.cache = {}

    def blocks(self, e, mat):
        key = (e, mat)
        if key not in self.cache:
            s = self.s
            shared = e == s.n_experts
            rows, cols = (s.inter, s.hidden) if mat in (0, 1) else (s.hidden, s.inter)
            fmt = s.fmt_shared if shared else (s.fmt_gate if mat in (0, 1) else s.fmt_down)
            self.cache[key] = (fmt, O.quantize_matrix(fmt, s.weight(e, mat, rows, cols)))
        return self.cache[key]

    def prefetch(self, experts, workers=8):
        keys = [(e, m) for e in experts for m in (0, 1, 2) if (e, m) not in self.cache]
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda km: self.blocks(*km), keys))

    def route(self, x, k):
        return O.route(x, self.s.router_w, self.s.router_b, k)

    def down_abs(self, e):
        """|dequantized down matrix| of expert e, fp64 [hidden][inter]."""
        key = ("absdown", e)
        if key not in self.cache:
            fmt, blk = self.blocks(e, 2)
            self.cache[key] = np.abs(O.dequantize_matrix(fmt, blk))
        return self.cache[key]

    def requant_bound(self, q, k, idx, w, hq_a, hs_a, hq_b, hs_b):
        """Elementwise bound on |y_a - y_b| for two runs of the down +
        combine stage that differ only in their requantized h (h~ = hs x hq
        per 32-block): y = sum_p w_p . Wd_p . h~_p, so |y_a - y_b| <=
        sum_p |w_p| . |Wd_p| . |h~_a,p - h~_b,p| (p over routed pairs, then
        the shared expert per token with weight 1). Returns fp64 [q][hidden]
        and the number of elements of h~ that differ."""
        s = self.s
        bound = np.zeros((q, s.hidden))
        n_diff = 0
        pairs = [(t * k + j, int(idx[t][j]), float(w[t][j]), t) for t in range(q) for j in range(k)]
        if s.shared:
            pairs += [(q * k + t, s.n_experts, 1.0, t) for t in range(q)]
        for p, e, wp, t in pairs:
            da = np.repeat(hs_a[p].astype(np.float64), 32) * hq_a[p].astype(np.float64)
            db = np.repeat(hs_b[p].astype(np.float64), 32) * hq_b[p].astype(np.float64)
            diff = np.abs(da - db)
            if np.any(diff > 0):
                bound[t] += abs(wp) * (self.down_abs(e) @ diff)
                n_diff += int(np.count_nonzero(diff))
        return bound, n_diff

    def expert_ffn(self, e, xq, xs, hq_override=None):
        fg, gb = self.blocks(e, 0)
        fu, ub = self.blocks(e, 1)
        fd, db = self.blocks(e, 2)
        return O.ffn(fg, gb, fu, ub, fd, db, xq, xs, hq_override)

    def layer(self, x, k, idx, w, hq_gpu=None, hs_gpu=None):
        """y (fp64) for tokens x with the given routing. With hq_gpu/hs_gpu
        ([q*k + q][I]) the down projections take the GPU's h~ instead of the
        oracle's own. Returns y, h [q*k+q][I], hq, hs."""
        s = self.s
        q = x.shape[0]
        xq, xs = O.quantize_act(x)
        NP = q * k + q
        h = np.zeros((NP, s.inter))
        hq = np.zeros((NP, s.inter), np.int8)
        hs = np.zeros((NP, s.inter // 32), np.float32)
        o = np.zeros((NP, s.hidden))
        jobs = []
        for t in range(q):
            for j in range(k):
                jobs.append((t * k + j, int(idx[t][j]), t))
            if s.shared:
                jobs.append((q * k + t, s.n_experts, t))
        for p, e, t in jobs:
            ov = None
            if hq_gpu is not None:
                ov = (hq_gpu[p:p + 1], hs_gpu[p:p + 1])
            r = self.expert_ffn(e, xq[t:t + 1], xs[t:t + 1], ov)
            h[p], hq[p], hs[p], o[p] = r["h"][0], r["hq"][0], r["hs"][0], r["o"][0]
        o_sh = o[q * k:] if s.shared else np.zeros((q, s.hidden))
        y = O.combine(o_sh, o[:q * k].reshape(q, k, s.hidden), w)
        return y, h, hq, hs


def check_routing(x, k, gpu, ref, delta_rel=1e-4):
    """Router indices bit-exact except where the fp64 logits sit within
    delta of each other at the selection boundary or inside the top-k;
    there the GPU's choice must be one of the tied orders. Returns the
    number of near-tie tokens."""
    idx_g = gpu["topk_idx"]
    near = 0
    for t in range(x.shape[0]):
        l = ref["logits"][t]
        order = ref["idx"][t]
        g = idx_g[t]
        if np.array_equal(g, order):
            continue
        # all GPU-chosen logits must be within delta of the oracle's k-th
        # best, every unchosen one must not beat a chosen one by > delta
        kth = np.sort(l)[::-1][k - 1]
        tol = delta_rel * (1.0 + abs(kth))
        chosen = l[g]
        rest = np.delete(l, g)
        assert np.all(chosen >= kth - tol), (t, g, order)
        assert np.all(rest <= chosen.min() + tol), (t, g, order)
        assert np.all(np.diff(chosen) <= tol), (t, g, order)
        assert len(set(g.tolist())) == k
        near += 1
    return near
