"""Host helpers that build an MoE layer in device memory and hold the
per-call buffers. Weights come from any provider of fp32 matrices; they are
quantized with the library's host encoder (rfx_quantize_matrix) and copied
to the GPU once."""

from __future__ import annotations

import ctypes
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (FP2, FP3, FP4, DeviceQMat, MoeLayerC, QMat, lib, moe_workspace_bytes,
               qmat_bytes, quantize_matrix)

GATE, UP, DOWN = 0, 1, 2


class DeviceMoeLayer:
    """Routed expert stacks (gate/up: inter x hidden, down: hidden x inter),
    an optional shared expert, and fp32 router weights/bias on the GPU."""

    def __init__(self, hidden, inter, n_experts, gate, up, down, sh=None, router_w=None,
                 router_b=None):
        self.hidden, self.inter, self.n_experts = hidden, inter, n_experts
        self.gate, self.up, self.down = gate, up, down
        self.sh = sh  # (gate, up, down) DeviceQMat or None
        self.router_w, self.router_b = router_w, router_b
        z = QMat(0, 0, 0, 0, None)
        c = MoeLayerC()
        c.hidden, c.inter, c.n_experts = hidden, inter, n_experts
        c.gate, c.up, c.down = gate.c, up.c, down.c
        if sh is not None:
            c.sh_gate, c.sh_up, c.sh_down = sh[0].c, sh[1].c, sh[2].c
        else:
            c.sh_gate = c.sh_up = c.sh_down = z
        c.router_w = router_w.data_ptr()
        c.router_b = router_b.data_ptr() if router_b is not None else None
        self.c = c

    def ref(self):
        return ctypes.byref(self.c)

    @classmethod
    def build(cls, hidden, inter, n_experts, weight_fn, router_w, router_b=None,
              fmt_gate=FP2, fmt_down=FP3, fmt_shared=FP4, shared=True, workers=8,
              device="cuda"):
        """weight_fn(expert, mat, rows, cols) -> fp32 [rows][cols]; mat is
        0 gate, 1 up, 2 down; expert == n_experts asks for the shared one."""
        import torch

        def stack(fmt, rows, cols, mat, count, first):
            nb = qmat_bytes(fmt, rows, cols)
            host = np.empty(count * nb, np.uint8)

            def one(e):
                W = weight_fn(first + e, mat, rows, cols)
                quantize_matrix(fmt, W, threads=1, out=host[e * nb:(e + 1) * nb])

            if count == 1:
                one(0)
            else:
                with ThreadPoolExecutor(workers) as ex:
                    list(ex.map(one, range(count)))
            return DeviceQMat(fmt, rows, cols, torch.from_numpy(host).to(device), count)

        gate = stack(fmt_gate, inter, hidden, GATE, n_experts, 0)
        up = stack(fmt_gate, inter, hidden, UP, n_experts, 0)
        down = stack(fmt_down, hidden, inter, DOWN, n_experts, 0)
        sh = None
        if shared:
            sh = (stack(fmt_shared, inter, hidden, GATE, 1, n_experts),
                  stack(fmt_shared, inter, hidden, UP, 1, n_experts),
                  stack(fmt_shared, hidden, inter, DOWN, 1, n_experts))
        rw = torch.from_numpy(np.ascontiguousarray(router_w, np.float32)).to(device)
        rb = None
        if router_b is not None:
            rb = torch.from_numpy(np.ascontiguousarray(router_b, np.float32)).to(device)
        return cls(hidden, inter, n_experts, gate, up, down, sh, rw, rb)

    def weight_bytes(self, experts, with_shared=True, with_router=True) -> int:
        """Packed bytes streamed for the given set of routed experts."""
        per = (qmat_bytes(self.gate.fmt, self.inter, self.hidden) * 2 +
               qmat_bytes(self.down.fmt, self.hidden, self.inter))
        n = per * len(set(int(e) for e in experts))
        if with_shared and self.sh is not None:
            n += (qmat_bytes(self.sh[0].fmt, self.inter, self.hidden) * 2 +
                  qmat_bytes(self.sh[2].fmt, self.hidden, self.inter))
        if with_router:
            n += self.n_experts * self.hidden * 4
        return n


def hot_experts_by_frequency(counts, n_hot):
    """The n_hot experts picked most often (ties to the lower id): the
    placement policy for a fixed budget of expert slots in HBM. counts: picks
    per expert from a warm-up run or the router's known bias."""
    counts = np.asarray(counts)
    order = np.lexsort((np.arange(len(counts)), -counts))
    return sorted(int(e) for e in order[:n_hot])


class PlacedMoeLayer(DeviceMoeLayer):
    """The experts of a DeviceMoeLayer placed by temperature: routed experts
    in `hot` stay in device memory (HBM), the others move to pinned host
    memory, which the kernels read directly over the host link; a device
    table of per-expert pointers ([gate e][up e][down e]) tells the kernels
    where each is (rfx_moe_layer.expert_data). The shared expert and the
    router stay in device memory."""

    def __init__(self, layer: DeviceMoeLayer, hot, device="cuda"):
        import torch
        E = layer.n_experts
        self.hot = sorted(set(int(e) for e in hot))
        hot_set = set(self.hot)
        self.cold = [e for e in range(E) if e not in hot_set]
        mats = (layer.gate, layer.up, layer.down)
        table = np.zeros((3, E), np.uint64)
        self.hot_data, self.cold_data = [], []
        for m, qm in enumerate(mats):
            nb = qmat_bytes(qm.fmt, qm.rows, qm.cols)
            hot_t = torch.empty(max(1, len(self.hot)) * nb, dtype=torch.uint8, device=device)
            cold_t = torch.empty(max(1, len(self.cold)) * nb, dtype=torch.uint8, pin_memory=True)
            for i, e in enumerate(self.hot):
                hot_t[i * nb:(i + 1) * nb].copy_(qm.data[e * nb:(e + 1) * nb])
                table[m, e] = hot_t.data_ptr() + i * nb
            for i, e in enumerate(self.cold):
                cold_t[i * nb:(i + 1) * nb].copy_(qm.data[e * nb:(e + 1) * nb])
                table[m, e] = cold_t.data_ptr() + i * nb
            self.hot_data.append(hot_t)
            self.cold_data.append(cold_t)
        torch.cuda.synchronize()
        self.table = torch.from_numpy(table.view(np.int64)).to(device)
        z = [DeviceQMat(qm.fmt, qm.rows, qm.cols, None, qm.count) for qm in mats]
        super().__init__(layer.hidden, layer.inter, E, z[0], z[1], z[2], layer.sh, layer.router_w, layer.router_b)
        self.c.expert_data = self.table.data_ptr()
        self.source = layer

    def hbm_bytes(self):
        """Packed routed-expert bytes held in device memory and in host memory."""
        per = sum(qmat_bytes(qm.fmt, qm.rows, qm.cols) for qm in (self.gate, self.up, self.down))
        return per * len(self.hot), per * len(self.cold)


class MoeBuffers:
    """Device buffers for one MoE decode call with q tokens, top-k."""

    def __init__(self, layer: DeviceMoeLayer, q: int, k: int, device="cuda"):
        import torch
        H, E = layer.hidden, layer.n_experts
        self.q, self.k = q, k
        self.topk_idx = torch.empty((q, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((q, k), dtype=torch.float32, device=device)
        self.pairs_sorted = torch.empty(q * k, dtype=torch.int32, device=device)
        self.expert_off = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.xq = torch.empty((q, H), dtype=torch.int8, device=device)
        self.xs = torch.empty((q, H // 32), dtype=torch.float32, device=device)
        self.xsum = torch.empty((q, H // 32), dtype=torch.int32, device=device)
        self.y = torch.empty((q, H), dtype=torch.float32, device=device)
        self.ws = torch.zeros(moe_workspace_bytes(layer, q, k), dtype=torch.uint8, device=device)

    def forward(self, layer: DeviceMoeLayer, x, resid=None, out=None, one_launch=False, stream=None):
        """The same as run(), through rfx_moe_forward: at q <= 4 the router
        launch computes the logits and every gate/up workgroup picks the top
        k itself (one_launch: the single-launch layer kernel for the page's
        formats instead)."""
        from . import moe_forward
        y = self.y if out is None else out
        moe_forward(layer, x, self.q, self.k, y, self.topk_idx, self.topk_w, self.pairs_sorted, self.expert_off,
                    self.xq, self.xs, self.xsum, self.ws, resid, one_launch, stream)
        return y

    def run(self, layer: DeviceMoeLayer, x, resid=None, out=None, stream=None):
        """route + FFN for x (device fp32 [q][hidden]); y = resid + MoE(x)
        lands in `out` (default self.y)."""
        from . import moe_ffn, moe_route_topk
        y = self.y if out is None else out
        moe_route_topk(layer, x, self.q, self.k, self.topk_idx, self.topk_w, self.pairs_sorted,
                       self.expert_off, self.xq, self.xs, self.xsum, self.ws, stream)
        moe_ffn(layer, self.q, self.k, self.xq, self.xs, self.xsum, self.topk_idx, self.topk_w,
                self.pairs_sorted, self.expert_off, y, self.ws, resid, stream)
        return y
