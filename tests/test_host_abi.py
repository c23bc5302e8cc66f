"""CPU tests of librfx's host side: the library loads and exports every
symbol the header declares; the host encoder and the tiled packer agree
bit for bit with the oracle; argument validation fails before any HIP call.
No GPU is touched."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FMTS = (2, 3, 4)
# the named formats, the FP2M variant, the Q8 tier, the FP2S variant, the FP3E tier
ALL_FMTS = (2, 3, 4, 12, 8, 16, 13)


def _header_functions():
    src = open(os.path.join(ROOT, "include", "rfx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rfx_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = R.lib()
    names = _header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(R.EXPORTED)
    assert R.lib().rfx_version().decode().startswith("rfx")


def test_sizes():
    for fmt, (bb, cb, sb, tile) in {2: (10, 8, 2, 5120), 3: (14, 12, 2, 7168),
                                     4: (17, 16, 1, 8704), 12: (12, 8, 4, 6144),
                                     8: (34, 32, 2, 17408), 16: (12, 8, 4, 6144),
                                     13: (13, 12, 1, 6656)}.items():
        assert R.block_bytes(fmt) == bb == O.block_bytes(fmt)
        assert R.code_bytes(fmt) == cb and R.scale_bytes(fmt) == sb
        assert R.qmat_bytes(fmt, 64, 256) == tile == 64 * 8 * bb
        assert R.qmat_bytes(fmt, 65, 288) == 4 * tile
    assert R.block_bytes(5) == -1


def _adversarial_blocks():
    rng = np.random.default_rng(77)
    blocks = []
    for k in range(400):
        w = (rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
        blocks.append(w)
    # exact ties for every format: amax fixes s = 1 (FP2: 3, FP3: 7), FP4 S = 1/2
    for amax, grid in ((3.0, [2.0, -2.0, 0.0, -0.0, 1.0, 2.5]),
                       (7.0, [2.0, 4.0, 6.0, -2.0, -4.0, -6.0, 0.0, -0.0]),
                       (6.0, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.25, -2.5, -3.5])):
        w = np.zeros(32, np.float32)
        w[0] = amax
        w[1:1 + len(grid)] = grid
        blocks.append(w)
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, 1e-9, np.float32))     # fp16 scale underflow
    blocks.append(np.full(32, 3e-6, np.float32))     # subnormal fp16 scale
    blocks.append(np.full(32, -2.0 ** -140, np.float32))  # subnormal weights
    w = np.zeros(32, np.float32)
    w[7] = 2.0 ** -130
    blocks.append(w)
    # FP2M: exact ties (m = 0, s = 1), a minimum that rounds above every
    # weight (negative span), signed zeros in either order, an offset block
    w = np.zeros(32, np.float32)
    w[1:6] = [3.0, 0.5, 1.5, 2.5, 1.0]
    blocks.append(w)
    blocks.append(np.full(32, 0.99995, np.float32))
    for first in (-0.0, 0.0):
        w = np.zeros(32, np.float32)
        w[0] = first
        w[5] = -first
        blocks.append(w)
    blocks.append((rng.standard_normal(32) * 0.01 + 40.0).astype(np.float32))
    blocks.append(np.linspace(-65000.0, 60000.0, 32).astype(np.float32))
    # FP2S: halves on scales 2^33 apart, one half zero, one half underflowing
    # to a zero fp16 scale, exact ties in the second half only
    blocks.append(np.r_[np.full(16, 1e-6), np.full(16, 1e4)].astype(np.float32))
    blocks.append(np.r_[np.zeros(16), rng.standard_normal(16)].astype(np.float32))
    blocks.append(np.r_[np.full(16, 1e-9), rng.standard_normal(16)].astype(np.float32))
    w = np.zeros(32, np.float32)
    w[16:22] = [3.0, 2.0, -2.0, 0.0, -0.0, 1.0]
    w[0] = 0.7
    blocks.append(w)
    return blocks


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_host_encoder_matches_oracle(fmt):
    for w in _adversarial_blocks():
        a = R.quantize_block(fmt, w)
        b = O.quantize_block(fmt, w)
        assert bytes(a) == bytes(b), (fmt, w)
        # the host decoder returns fp32: exact for s * v (an fp16 times a
        # small integer); FP2M's s * c + m is the fp32 rounding of the exact
        # value (one rounding, the product being exact)
        ref = O.dequantize_block(fmt, b)
        if fmt == 12:
            ref = ref.astype(np.float32).astype(np.float64)
        assert np.array_equal(R.dequantize_block(fmt, a).astype(np.float64), ref)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("shape", [(1, 32), (64, 256), (65, 288), (200, 544), (130, 1024)])
def test_tiled_packer_roundtrip(fmt, shape):
    rows, cols = shape
    W = inputgen.dense_weight(rows, cols, seed=rows + cols, outliers=True)
    t = R.quantize_matrix(fmt, W, threads=3)
    assert t.nbytes == R.qmat_bytes(fmt, rows, cols)
    blocks = R.export_blocks(fmt, t, rows, cols)
    assert np.array_equal(blocks, O.quantize_matrix(fmt, W))
    assert np.array_equal(R.import_blocks(fmt, blocks), t)


def test_tiled_layout_positions():
    """A block's bytes land where the header says: tile (g, s), chunk c,
    row r at c*1024 + r*16."""
    rows, cols = 130, 600
    for fmt in ALL_FMTS:
        nb = cols // 32
        bb = R.block_bytes(fmt)
        blocks = np.zeros((rows, nb, bb), np.uint8)
        r, b = 70, 9  # g = 1, lane 6, s = 1, bi = 1
        blocks[r, b] = np.arange(1, bb + 1, dtype=np.uint8)
        t = R.import_blocks(fmt, blocks)
        S = -(-cols // 256)
        tile = (1 * S + 1) * R.qmat_bytes(fmt, 64, 256)
        lane, bi = 6, 1
        if fmt == 4:
            assert list(t[tile + bi * 1024 + lane * 16: tile + bi * 1024 + lane * 16 + 16]) == list(range(1, 17))
            assert t[tile + 8192 + lane * 8 + bi] == 17
        elif fmt == 13:  # FP3's code chunks, then one e8m0 byte per block
            c0 = tile + (bi // 2) * 1024 + lane * 16 + (bi % 2) * 8
            assert list(t[c0:c0 + 8]) == list(range(1, 9))
            c1 = tile + (4 + bi // 4) * 1024 + lane * 16 + (bi % 4) * 4
            assert list(t[c1:c1 + 4]) == [9, 10, 11, 12]
            assert t[tile + 6144 + lane * 8 + bi] == 13
        elif fmt == 8:
            for h in range(2):
                c = tile + (2 * bi + h) * 1024 + lane * 16
                assert list(t[c:c + 16]) == list(range(1 + 16 * h, 17 + 16 * h))
            sc = tile + 16 * 1024 + lane * 16 + bi * 2
            assert list(t[sc:sc + 2]) == [33, 34]
        else:
            c0 = tile + (bi // 2) * 1024 + lane * 16 + (bi % 2) * 8
            assert list(t[c0:c0 + 8]) == list(range(1, 9))
            if fmt == 3:
                c1 = tile + (4 + bi // 4) * 1024 + lane * 16 + (bi % 4) * 4
                assert list(t[c1:c1 + 4]) == [9, 10, 11, 12]
                sc = tile + 6 * 1024 + lane * 16 + bi * 2
                assert list(t[sc:sc + 2]) == [13, 14]
            else:
                sc = tile + 4 * 1024 + lane * 16 + bi * 2
                assert list(t[sc:sc + 2]) == [9, 10]
                if fmt in (12, 16):  # FP2M's minimum, FP2S's second scale
                    mn = tile + 5 * 1024 + lane * 16 + bi * 2
                    assert list(t[mn:mn + 2]) == [11, 12]
        assert int(t.astype(np.int64).sum()) == int(np.arange(1, bb + 1).sum())


def test_encoder_errors():
    w = np.zeros(32, np.float32)
    w[0] = np.nan
    with pytest.raises(R.RfxError) as e:
        R.quantize_block(2, w)
    assert e.value.status == -3
    with pytest.raises(R.RfxError):
        R.quantize_block(2, np.full(32, 3e5, np.float32))
    with pytest.raises(R.RfxError) as e:
        R.quantize_matrix(9, np.zeros((4, 32), np.float32))
    assert e.value.status == -1
    with pytest.raises(R.RfxError):
        R.quantize_matrix(2, np.zeros((4, 40), np.float32))
    W = np.zeros((70, 64), np.float32)
    W[69, 3] = np.inf
    with pytest.raises(R.RfxError) as e:
        R.quantize_matrix(3, W, threads=4)
    assert e.value.status == -3


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_device_entry_validation_without_gpu():
    """Every check runs before the first HIP call."""
    L = R.lib()
    good = 0x7f0000000000  # aligned fake address; never dereferenced
    W = R.QMat(2, 128, 512, 1, good)
    null = None
    st = L.rfx_gemv(None, _fake(good), _fake(good), _fake(good), 1, _fake(good), null, 0, null)
    assert st == -1
    st = L.rfx_gemv(ctypes.byref(W), _fake(good), _fake(good), _fake(good), 5, _fake(good), null, 0, null)
    assert st == -1
    st = L.rfx_gemv(ctypes.byref(W), None, _fake(good), _fake(good), 1, _fake(good), null, 0, null)
    assert st == -1
    st = L.rfx_gemv(ctypes.byref(W), _fake(good + 1), _fake(good), _fake(good), 1, _fake(good), null, 0, null)
    assert st == -2
    bad = R.QMat(2, 128, 500, 1, good)
    assert L.rfx_gemv(ctypes.byref(bad), _fake(good), _fake(good), _fake(good), 1, _fake(good), null, 0, null) == -1
    mis = R.QMat(2, 128, 512, 1, good + 16)
    assert L.rfx_gemv(ctypes.byref(mis), _fake(good), _fake(good), _fake(good), 1, _fake(good), null, 0, null) == -2
    stack = R.QMat(2, 128, 512, 3, good)
    assert L.rfx_gemv(ctypes.byref(stack), _fake(good), _fake(good), _fake(good), 1, _fake(good), null, 0, null) == -1
    # split-K workspace too small -> RFX_E_WORKSPACE, still before HIP
    big = R.QMat(4, 7168, 7168, 1, good)
    need = L.rfx_gemv_workspace_bytes(ctypes.byref(big), 4)
    assert need > 0
    st = L.rfx_gemv(ctypes.byref(big), _fake(good), _fake(good), _fake(good), 4, _fake(good),
                    _fake(good), need - 4, null)
    assert st == -5
    # grouped GEMV: job count, a bad job (named by index), workspace size
    f = _fake(good).value
    jobs = (R.GemvJob * 3)(*[R.GemvJob(R.QMat(fmt, 7168, 7168, 1, good), q, 0, f, f, f, f)
                             for fmt, q in ((2, 1), (3, 4), (4, 2))])
    assert L.rfx_gemv_grouped(jobs, 0, null, 0, null) == -1
    assert L.rfx_gemv_grouped(jobs, 17, null, 0, null) == -1
    assert L.rfx_gemv_grouped(None, 1, null, 0, null) == -1
    need = L.rfx_gemv_grouped_workspace_bytes(jobs, 3)
    assert need >= 3 * 256 and need % 256 == 0
    assert L.rfx_gemv_grouped(jobs, 3, _fake(good), need - 256, null) == -5
    assert L.rfx_gemv_grouped(jobs, 3, None, need, null) == -5
    jobs[1].q = 5
    assert L.rfx_gemv_grouped(jobs, 3, _fake(good), need, null) == -1
    assert b"jobs[1]" in L.rfx_last_error()
    jobs[1].q = 4
    jobs[2].xq = good + 4
    assert L.rfx_gemv_grouped(jobs, 3, _fake(good), need, null) == -2
    assert b"jobs[2]" in L.rfx_last_error()
    jobs[2].xq = f
    jobs[0].W.cols = 7000
    assert L.rfx_gemv_grouped(jobs, 3, _fake(good), need, null) == -1
    assert b"jobs[0]" in L.rfx_last_error()
    assert L.rfx_quantize_act(_fake(good), 1, 40, _fake(good), _fake(good), _fake(good), null) == -1
    assert L.rfx_quantize_act(None, 1, 64, _fake(good), _fake(good), _fake(good), null) == -1
    # x and xq are read and written 16 bytes at a time
    assert L.rfx_quantize_act(_fake(good + 4), 1, 64, _fake(good), _fake(good), _fake(good), null) == -2
    assert L.rfx_quantize_act(_fake(good), 1, 64, _fake(good + 8), _fake(good), _fake(good), null) == -2
    assert L.rfx_debug_block_dots(ctypes.byref(W), _fake(good), _fake(good), 0, _fake(good), null) == -1
    assert b"q" in L.rfx_last_error()
    # the no-workspace GEMV validates the same way, before looking up its scratch
    assert L.rfx_gemv_noalloc(None, _fake(good), _fake(good), _fake(good), 1, _fake(good), null) == -1
    assert L.rfx_gemv_noalloc(ctypes.byref(W), _fake(good), _fake(good), _fake(good), 5, _fake(good), null) == -1
    assert L.rfx_gemv_noalloc(ctypes.byref(W), _fake(good + 1), _fake(good), _fake(good), 1, _fake(good), null) == -2
    assert L.rfx_gemv_noalloc(ctypes.byref(stack), _fake(good), _fake(good), _fake(good), 1, _fake(good), null) == -1


def test_moe_rejects_the_gemv_only_variant():
    """The MoE and prefill layers refuse FP2M and FP2S before any HIP call."""
    L = R.lib()
    good = 0x7f0000000000
    f = _fake(good)
    H, I, E = 256, 512, 4
    lay = R.MoeLayerC(H, I, E, 0, R.QMat(12, I, H, E, good), R.QMat(12, I, H, E, good),
                      R.QMat(3, H, I, E, good), R.QMat(0, 0, 0, 0, None), R.QMat(0, 0, 0, 0, None),
                      R.QMat(0, 0, 0, 0, None), good, None)
    st = L.rfx_moe_ffn(ctypes.byref(lay), 1, 2, f, f, f, f, f, f, f, f, f, f, 1 << 20, None)
    assert st == -4 and b"FP2M" in L.rfx_last_error()
    lay.gate.fmt = lay.up.fmt = 2
    lay.down.fmt = 12
    st = L.rfx_moe_route_topk(ctypes.byref(lay), f, 1, 2, f, f, f, f, f, f, f, f, 1 << 20, None)
    assert st == -4
    for fmt in (16, 13):
        lay.down.fmt = fmt
        st = L.rfx_moe_ffn(ctypes.byref(lay), 1, 2, f, f, f, f, f, f, f, f, f, f, 1 << 20, None)
        assert st == -4 and b"FP3E" in L.rfx_last_error()


def test_moe_debug_hooks_validation_without_gpu():
    """The MoE test hooks check the workspace size against the q and k they
    are given (and the prefill hook its q and probe) before any HIP call."""
    L = R.lib()
    good = 0x7f0000000000
    f = _fake(good)
    H, I, E = 256, 512, 4
    z = R.QMat(0, 0, 0, 0, None)
    lay = R.MoeLayerC(H, I, E, 0, R.QMat(2, I, H, E, good), R.QMat(2, I, H, E, good),
                      R.QMat(3, H, I, E, good), z, z, z, good, None)
    need = L.rfx_moe_workspace_bytes(ctypes.byref(lay), 4, 2)
    assert need > 0
    assert L.rfx_moe_debug_hidden(ctypes.byref(lay), 4, 2, f, need - 256, f, f, f, None) == -5
    assert L.rfx_moe_debug_hidden(ctypes.byref(lay), 4, 3, f, need, None, f, f, None) == -5  # larger k
    assert L.rfx_moe_debug_hidden(ctypes.byref(lay), 4, 2, None, need, None, f, f, None) == -1
    need_p = L.rfx_moe_workspace_bytes(ctypes.byref(lay), 64, 2)

    def pre(q, ws_bytes, pe, pf):
        return L.rfx_moe_debug_prefill(ctypes.byref(lay), q, 2, f, f, f, f, f, f, ws_bytes, pe, pf,
                                       f, f, f, f, None)

    assert pre(4, need_p, 0, 0) == -1          # the decode sizes have no prefill kernels
    assert pre(64, need_p - 256, 0, 0) == -5
    assert pre(64, need_p, E, 0) == -1         # no shared expert in this layer
    assert pre(64, need_p, -1, 0) == -1
    assert pre(64, need_p, 0, 3) == -1         # a work item starts at a multiple of 64
    assert L.rfx_moe_debug_prefill(ctypes.byref(lay), 64, 2, _fake(good + 4), f, f, f, f, f, need_p, 0, 0,
                                   f, f, f, f, None) == -2


def test_moe_forward_validation_without_gpu():
    """rfx_moe_forward checks what both of its calls check before any HIP
    call; rfx_moe_forward_single_launch is host logic: one launch for q <= 4
    with FP2 gate/up, FP3 down and an FP4 shared expert (or none), two calls
    otherwise."""
    L = R.lib()
    good = 0x7f0000000000
    f = _fake(good)
    H, I, E = 512, 256, 16
    z = R.QMat(0, 0, 0, 0, None)

    def layer(fg, fd, fs):
        sh = [R.QMat(fs, I, H, 1, good), R.QMat(fs, I, H, 1, good), R.QMat(fs, H, I, 1, good)] if fs else [z, z, z]
        return R.MoeLayerC(H, I, E, 0, R.QMat(fg, I, H, E, good), R.QMat(fg, I, H, E, good),
                           R.QMat(fd, H, I, E, good), *sh, good, None, None)

    lay = layer(2, 3, 4)
    for q in (1, 2, 3, 4):
        assert L.rfx_moe_forward_single_launch(ctypes.byref(lay), q, 4) == 1
    assert L.rfx_moe_forward_single_launch(ctypes.byref(lay), 5, 4) == 0   # prefill sizes: two calls
    assert L.rfx_moe_forward_single_launch(ctypes.byref(layer(2, 3, 0)), 1, 8) == 1  # no shared expert
    for fmts in ((4, 3, 4), (2, 2, 4), (2, 3, 2), (3, 3, 4)):
        assert L.rfx_moe_forward_single_launch(ctypes.byref(layer(*fmts)), 1, 4) == 0
    assert L.rfx_moe_forward_single_launch(None, 1, 4) == -1
    assert L.rfx_moe_forward_single_launch(ctypes.byref(lay), 1, 9) == -1

    need = L.rfx_moe_workspace_bytes(ctypes.byref(lay), 2, 4)
    assert need > 0

    def fwd(lp, q, k, x=f, resid=None, ws=f, ws_bytes=need, flags=1):
        return L.rfx_moe_forward(lp, x, q, k, resid, f, f, f, f, f, f, f, f, ws, ws_bytes, flags, None)

    assert fwd(None, 2, 4) == -1
    assert fwd(ctypes.byref(lay), 2, 0) == -1
    assert fwd(ctypes.byref(lay), 0, 4) == -1
    assert fwd(ctypes.byref(lay), 2, 4, x=None) == -1
    assert fwd(ctypes.byref(lay), 2, 4, x=_fake(good + 4)) == -2
    assert fwd(ctypes.byref(lay), 2, 4, resid=_fake(good + 4)) == -2
    assert fwd(ctypes.byref(lay), 2, 4, ws=None) == -1
    assert fwd(ctypes.byref(lay), 2, 4, ws_bytes=need - 256) == -5
    assert fwd(ctypes.byref(lay), 3, 4) == -5   # sized for q = 2
    assert fwd(ctypes.byref(lay), 2, 4, flags=2) == -1
    assert fwd(ctypes.byref(lay), 2, 4, ws_bytes=need - 256, flags=0) == -5
    assert L.rfx_moe_forward_status(ctypes.byref(lay), 2, 4, f, need - 256, None) == -5
    assert L.rfx_moe_forward_status(ctypes.byref(lay), 2, 4, None, need, None) == -1


def test_read_reference_validation_without_gpu():
    L = R.lib()
    good = 0x7f0000000000
    f = _fake(good)
    assert L.rfx_read_reference(None, 64, f, 1, None) == -1
    assert L.rfx_read_reference(_fake(good + 8), 64, f, 1, None) == -2
    assert L.rfx_read_reference(f, 40, f, 1, None) == -1
    assert L.rfx_read_reference(f, 0, f, 1, None) == -1
    assert L.rfx_read_reference(f, 64, f, 0, None) == -1


def test_status_strings():
    L = R.lib()
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.rfx_status_str(st)
    assert L.rfx_status_str(-99) == b"unknown status"


def test_hot_expert_policy():
    """The n most picked experts, ties to the lower id."""
    from bit_block_quantized_amd.layer import hot_experts_by_frequency
    counts = np.array([5, 9, 9, 0, 7, 9, 1])
    assert hot_experts_by_frequency(counts, 3) == [1, 2, 5]
    assert hot_experts_by_frequency(counts, 4) == [1, 2, 4, 5]
    assert hot_experts_by_frequency(counts, 0) == []
    assert hot_experts_by_frequency(counts, 10) == list(range(7))


def test_placement_table_validation_without_gpu():
    """With a per-expert pointer table the routed stacks need no data
    pointer; the table itself must be present and 8-byte aligned."""
    L = R.lib()
    good = 0x7f0000000000
    f = _fake(good)
    H, I, E = 256, 512, 4
    z = R.QMat(0, 0, 0, 0, None)
    lay = R.MoeLayerC(H, I, E, 0, R.QMat(2, I, H, E, None), R.QMat(2, I, H, E, None),
                      R.QMat(3, H, I, E, None), z, z, z, good, None, None)
    need = L.rfx_moe_workspace_bytes(ctypes.byref(lay), 1, 2)
    assert L.rfx_moe_ffn(ctypes.byref(lay), 1, 2, f, f, f, f, f, f, f, f, f, f, need, None) == -1  # stacks NULL, no table
    lay.expert_data = good + 4
    assert L.rfx_moe_ffn(ctypes.byref(lay), 1, 2, f, f, f, f, f, f, f, f, f, f, need, None) == -2


def test_prefill_workspace_holds_the_f16_activation_copies():
    """The prefill FFN keeps f16 copies of the token codes ([q][H]) and of
    h~ ([q*k + q][I]) in the workspace; its size must cover them even where
    they exceed the fp32 h rows the decode path keeps (H > (k + 1) I)."""
    L = R.lib()
    good = 0x7f0000000000
    H, I, E, k = 4096, 256, 4, 1
    z = R.QMat(0, 0, 0, 0, None)
    lay = R.MoeLayerC(H, I, E, 0, R.QMat(2, I, H, E, good), R.QMat(2, I, H, E, good),
                      R.QMat(3, H, I, E, good), z, z, z, good, None)
    for q in (64, 2048):
        need = L.rfx_moe_workspace_bytes(ctypes.byref(lay), q, k)
        assert need >= q * H * 2 + (q * k + q) * I * 2 + (q * k + q) * I  # copies + int8 h~
    # the decode sizes keep fp32 h only
    assert L.rfx_moe_workspace_bytes(ctypes.byref(lay), 4, k) >= (4 * k + 4) * I * 4
