"""GPU parity of the activation quantizer and the fused block GEMV against
the CPU oracle: quantized activations and per-block integer dots bit-exact,
fp32 outputs within 1e-4 (floored relative), at small ragged shapes, at the
1024 x 1024 FP4 workload and at the 7168 x 7168 FP2/FP3/FP4 workloads in
the launch configuration the benchmark times (split-K with a workspace)."""

import numpy as np
import pytest

import bit_block_quantized_amd as R
import inputgen
import oracle as O
from gpu_common import TOL, need_gpu, quantize_on_gpu, rel_err, say, upload_matrix, workspace

pytestmark = pytest.mark.gpu
FMTS = (2, 3, 4)
FP2M = R.FP2M
Q8 = R.Q8
FP2S = R.FP2S
FP3E = R.FP3E
# the GEMV entry points also take the FP2M and FP2S variants and the Q8 and
# FP3E tiers
GEMV_FMTS = FMTS + (FP2M, Q8, FP2S, FP3E)


def _sync(torch):
    torch.cuda.synchronize()


# ------------------------------------------------------------ activations

@pytest.mark.parametrize("q,K", [(1, 32), (4, 544), (4, 7168), (3, 4096)])
def test_act_quant_bit_exact(q, K):
    torch = need_gpu()
    say(f"act_quant q={q} K={K}")
    x = inputgen.activations(q, K, seed=3) * np.float32(2.0)
    x[0, :32] = 0.0  # a zero block
    if K >= 64:  # exact rounding ties: amax 127 -> s = 1
        x[-1, 32] = 127.0
        x[-1, 33:63] = np.arange(-15, 15, dtype=np.float32) + np.float32(0.5)
    xq, xs, xsum = quantize_on_gpu(torch, x)
    _sync(torch)
    oq, os_ = O.quantize_act(x)
    assert np.array_equal(xq.cpu().numpy(), oq)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(xsum.cpu().numpy(), O.act_sums(oq))


# ------------------------------------------------------------------ gemv

def _run(torch, fmt, W, x, q, split, blocks=None):
    """Returns (y_gpu, dots_gpu, y_oracle, dots_oracle)."""
    N, K = W.shape
    dW = upload_matrix(torch, fmt, W)
    xq, xs, xsum = quantize_on_gpu(torch, x)
    y = torch.full((q, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = workspace(torch, R.gemv_workspace_bytes(dW, q)) if split else None
    R.gemv(dW, xq, xs, xsum, q, y, ws)
    dots = torch.full((q, N, K // 32), -(2 ** 31), dtype=torch.int32, device="cuda")
    R.debug_block_dots(dW, xq, xsum, q, dots)
    _sync(torch)
    if blocks is None:
        blocks = O.quantize_matrix(fmt, W)
    oq, os_ = O.quantize_act(x)
    yo, do = O.gemv(fmt, blocks, oq, os_, want_dots=True)
    return y.cpu().numpy(), dots.cpu().numpy(), yo, do


@pytest.mark.parametrize("fmt", GEMV_FMTS)
@pytest.mark.parametrize("q", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(200, 544), (64, 256), (1, 32), (65, 288), (130, 2080)])
def test_gemv_small_shapes(fmt, q, shape):
    torch = need_gpu()
    N, K = shape
    say(f"gemv small fmt={fmt} q={q} N={N} K={K}")
    W = inputgen.dense_weight(N, K, seed=N + K + fmt, outliers=True)
    x = inputgen.activations(q, K, seed=5)
    for split in (False, True):
        y, d, yo, do = _run(torch, fmt, W, x, q, split)
        assert np.array_equal(d, do)
        assert rel_err(y, yo) <= TOL, (split, rel_err(y, yo))


def test_gemv_fp4_1024_q1():
    """Dense FP4 1024 x 1024, W seed 0, one column seed 1."""
    torch = need_gpu()
    say("gemv fp4 1024x1024 q=1")
    W = inputgen.dense_weight(1024, 1024, seed=0)
    x = inputgen.activations(1, 1024, seed=1)
    y, d, yo, do = _run(torch, 4, W, x, 1, split=True)
    assert np.array_equal(d, do)
    assert rel_err(y, yo) <= TOL


_BIG = {}


def _big(fmt):
    if fmt not in _BIG:
        W = inputgen.dense_weight(7168, 7168, seed={2: 0, 3: 10, 4: 20, FP2M: 30, Q8: 40, FP2S: 50, FP3E: 60}[fmt], outliers=True)
        _BIG[fmt] = (W, O.quantize_matrix(fmt, W))
    return _BIG[fmt]


@pytest.mark.parametrize("fmt", GEMV_FMTS)
@pytest.mark.parametrize("q", [1, 4])
def test_gemv_7168_full(fmt, q):
    """7168 x 7168 with 1% outliers, q columns seeds 1..q, split-K launch."""
    torch = need_gpu()
    say(f"gemv 7168 fmt={fmt} q={q}")
    W, blocks = _big(fmt)
    x = inputgen.activations(q, 7168, seed=1)
    y, d, yo, do = _run(torch, fmt, W, x, q, split=True, blocks=blocks)
    assert np.array_equal(d, do)
    err = rel_err(y, yo)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


def test_gemv_7168_fp4_q2():
    """FP4 with two columns also runs on the block-scaled matrix core (one
    column pair): its block dots and y at the full 7168 x 7168 size."""
    torch = need_gpu()
    say("gemv 7168 fmt=4 q=2")
    W, blocks = _big(4)
    x = inputgen.activations(2, 7168, seed=1)
    y, d, yo, do = _run(torch, 4, W, x, 2, split=True, blocks=blocks)
    assert np.array_equal(d, do)
    err = rel_err(y, yo)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


# exponent classes of the FP4 matrix-core dot test: products that are fp32
# subnormals, ordinary ones, and the top of the e8m0 range
_E_TINY = (0, 1, 2, 3, 5, 10)
_E_NORMAL = (100, 115, 120, 124, 126, 127, 128, 130, 140, 200, 243)
_E_HUGE = (245, 250, 252, 253, 254)


@pytest.mark.parametrize("q", [1, 2])
@pytest.mark.parametrize("shape", [(100, 544), (64, 512)])
def test_fp4_matrix_core_dots_extreme_exponents(q, shape):
    """FP4 with one or two columns runs on the block-scaled matrix core,
    which applies each block's e8m0 exponent inside the product. Its block
    dots must equal the oracle's exactly over the exponent range: blocks
    whose products are fp32 subnormals (E near 0; row 0 holds only such
    blocks), ordinary blocks, and E up to 254 with codes and activations
    small enough that every partial product stays finite (one nonzero code
    of magnitude 0.5 or 1, activations 0 or 1). The blocks are written as
    canonical bytes: the encoder never emits E above 252 from fp32 weights.
    Ragged N and K (a partial row group and a partial tile) and full tiles."""
    torch = need_gpu()
    N, K = shape
    nb = K // 32
    say(f"fp4 matrix-core dots, extreme exponents, q={q} N={N} K={K}")
    rng = np.random.default_rng(7000 + 10 * q + N)
    blocks = np.zeros((N, nb, 17), np.uint8)
    cls = np.array([0 if n == 0 else b % 3 for n in range(N) for b in range(nb)]).reshape(N, nb)
    xq = rng.integers(-127, 128, (q, K)).astype(np.int8)
    for b in range(nb):
        if b % 3 == 2:
            xq[:, 32 * b:32 * b + 32] = rng.integers(0, 2, (q, 32))
    for n in range(N):
        for b in range(nb):
            c = cls[n, b]
            if c == 2:
                codes = np.zeros(32, np.int64)
                codes[rng.integers(32)] = rng.choice([1, 2, 9, 10])  # +-0.5, +-1 in E2M1
                E = _E_HUGE[(n + b) % len(_E_HUGE)]
            else:
                codes = rng.integers(0, 16, 32)
                table = _E_TINY if c == 0 else _E_NORMAL
                E = table[(n + 3 * b) % len(table)]
            blocks[n, b, :16] = O.pack_codes(4, codes)
            blocks[n, b, 16] = E
    dW = R.DeviceQMat.from_host(4, N, K, R.import_blocks(4, blocks))
    xqd = torch.from_numpy(xq).cuda()
    xsumd = torch.from_numpy(O.act_sums(xq)).cuda()
    dots = torch.full((q, N, nb), -(2 ** 31), dtype=torch.int32, device="cuda")
    R.debug_block_dots(dW, xqd, xsumd, q, dots)
    _sync(torch)
    _, do = O.gemv(4, blocks, xq, np.ones((q, nb), np.float32), want_dots=True)
    d = dots.cpu().numpy()
    bad = d != do
    for c, name in enumerate(("tiny", "normal", "huge")):
        m = np.broadcast_to(cls == c, bad.shape)
        say(f"  {name} exponents: {int(bad[m].sum())} of {int(m.sum())} dots differ")
    assert not bad.any()


@pytest.mark.parametrize("fmt", GEMV_FMTS)
def test_gemv_deterministic_and_columns_independent(fmt):
    torch = need_gpu()
    say(f"gemv determinism fmt={fmt}")
    N, K = 7168, 4096
    W = inputgen.dense_weight(N, K, seed=11)
    dW = upload_matrix(torch, fmt, W)
    x = inputgen.activations(4, K, seed=12)
    xq, xs, xsum = quantize_on_gpu(torch, x)
    ws = workspace(torch, R.gemv_workspace_bytes(dW, 4))
    outs = []
    for _ in range(3):  # the same workspace reused: counters reset each call
        y = torch.empty((4, N), dtype=torch.float32, device="cuda")
        R.gemv(dW, xq, xs, xsum, 4, y, ws)
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # One column alone against the same column of the 4-column call. For
    # FP4 the two take different arithmetic (one or two columns: block dots
    # on the block-scaled matrix core, exponent applied inside the product;
    # more columns: vector decode and int8 dots), so they agree to fp32
    # rounding of the row sums rather than to the last bits; a column
    # leaking into another would be off by far more.
    same_path = fmt != 4  # FP4: matrix core at q = 1, vector path at q = 4
    oq, os_ = O.quantize_act(x)
    blocks = O.quantize_matrix(fmt, W)
    for j in range(4):
        ws1 = workspace(torch, R.gemv_workspace_bytes(dW, 1))
        y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
        R.gemv(dW, xq[j:j + 1], xs[j:j + 1], xsum[j:j + 1], 1, y1, ws1)
        err = rel_err(y1.cpu().numpy()[0], outs[0][j])
        say(f"  column {j}: q=1 vs q=4 rel diff {err:.2e}")
        assert err <= (1e-6 if same_path else 2e-5)
        if not same_path:
            yo = O.gemv(fmt, blocks, oq[j:j + 1], os_[j:j + 1])
            assert rel_err(y1.cpu().numpy()[0], yo[0]) <= TOL


@pytest.mark.parametrize("q", [1, 4])
def test_gemv_fp2m_offset_rows(q):
    """FP2M on rows whose weights sit far from zero (each row its own
    offset, the case the block minimum is for), with ragged K so the
    minimum of blocks past K must be dropped too."""
    torch = need_gpu()
    say(f"gemv fp2m offset rows q={q}")
    N, K = 300, 1312
    rng = np.random.default_rng(90 + q)
    W = (inputgen.dense_weight(N, K, seed=91) * np.float32(0.2)
         + rng.uniform(-3, 3, (N, 1)).astype(np.float32))
    x = inputgen.activations(q, K, seed=92)
    for split in (False, True):
        y, d, yo, do = _run(torch, FP2M, W, x, q, split)
        assert np.array_equal(d, do)
        assert rel_err(y, yo) <= TOL, (split, rel_err(y, yo))


@pytest.mark.parametrize("q", [1, 4])
def test_gemv_fp2s_halves_on_different_scales(q):
    """FP2S with the two halves of every block on scales 2^4 apart (the
    case the second scale is for; a half dot over the wrong weights or the
    scales swapped is far off), ragged K so both scales of blocks past K
    must be dropped."""
    torch = need_gpu()
    say(f"gemv fp2s half scales q={q}")
    N, K = 300, 1312
    W = inputgen.dense_weight(N, K, seed=95)
    W.reshape(N, K // 32, 32)[:, :, 16:] *= np.float32(16.0)
    x = inputgen.activations(q, K, seed=96)
    for split in (False, True):
        y, d, yo, do = _run(torch, FP2S, W, x, q, split)
        assert np.array_equal(d, do)
        assert rel_err(y, yo) <= TOL, (split, rel_err(y, yo))


def test_read_reference_folds_every_word():
    """The streaming-read reference (a measurement aid) reads every word:
    the XOR of its per-workgroup folds equals numpy's XOR of the buffer,
    including a size that leaves a remainder after the 4-load loop."""
    torch = need_gpu()
    say("read reference")
    rng = np.random.default_rng(3)
    for n_words, n_out in ((4 * 1000, 7), (4 * 65537, 64), (1 << 22, 512)):
        host = rng.integers(0, 2 ** 32, n_words, dtype=np.uint64).astype(np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda()
        out = torch.zeros(n_out, dtype=torch.int32, device="cuda")
        R.read_reference(buf, out)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), (n_words, n_out)


# ---------------------------------------------------------- grouped gemv

def _grouped(torch, specs, seed, big=False):
    """specs [(fmt, q, N, K)] through one rfx_gemv_grouped launch, twice on
    the same workspace; returns [(y_gpu_call1, y_gpu_call2, y_oracle)]."""
    jobs, refs = [], []
    for i, (fmt, q, N, K) in enumerate(specs):
        if big:
            W, blocks = _big(fmt)
        else:
            W = inputgen.dense_weight(N, K, seed=seed + i, outliers=True)
            blocks = O.quantize_matrix(fmt, W)
        x = inputgen.activations(q, K, seed=seed + 100 + i)
        xq, xs, xsum = quantize_on_gpu(torch, x)
        y = torch.full((q, N), float("nan"), dtype=torch.float32, device="cuda")
        jobs.append((upload_matrix(torch, fmt, W), q, xq, xs, xsum, y))
        oq, os_ = O.quantize_act(x)
        refs.append(O.gemv(fmt, blocks, oq, os_))
    arr = R.gemv_jobs(jobs)
    ws = workspace(torch, R.gemv_grouped_workspace_bytes(arr))
    R.gemv_grouped(arr, ws)
    _sync(torch)
    first = [j[5].cpu().numpy().copy() for j in jobs]
    for j in jobs:
        j[5].fill_(float("nan"))
    R.gemv_grouped(arr, ws)  # the workspace must come back zeroed
    _sync(torch)
    if ws is not None:
        assert int(ws.count_nonzero()) == 0
    return [(a, j[5].cpu().numpy(), r) for a, j, r in zip(first, jobs, refs)]


@pytest.mark.parametrize("specs", [
    # mixed formats and q, ragged N and K (partial tiles: K % 256 != 0)
    [(2, 1, 200, 544), (3, 4, 65, 288), (4, 2, 130, 2080), (2, 3, 1, 32), (4, 4, 64, 256)],
    # every K a multiple of 256 (the straight-line full-tile code), split K
    [(4, 1, 1024, 1024), (2, 4, 300, 4096), (3, 2, 77, 2048), (4, 3, 512, 768)],
    # a single job
    [(3, 4, 640, 1536)],
    # the FP2M variant beside the named formats, ragged and full tiles
    [(12, 1, 200, 544), (2, 4, 130, 2080), (12, 4, 65, 1024), (12, 2, 1, 32), (4, 1, 256, 512)],
    # the Q8 tier (one tile buffer) beside the others, a multi-tile K split
    [(8, 1, 300, 4096), (8, 4, 65, 1312), (3, 2, 130, 2048), (8, 3, 1, 32)],
    # the FP2S variant beside the others, ragged and full tiles
    [(16, 1, 200, 544), (16, 4, 130, 2080), (12, 2, 65, 1024), (16, 3, 1, 32), (2, 4, 256, 512)],
    # the FP3E tier beside FP3 (same code chunks, different scale area)
    [(13, 1, 300, 4096), (3, 1, 300, 4096), (13, 4, 65, 1312), (13, 2, 1, 32), (4, 3, 130, 2080)],
])
def test_gemv_grouped_small(specs):
    torch = need_gpu()
    say(f"gemv grouped {specs}")
    for i, (a, b, ref) in enumerate(_grouped(torch, specs, seed=40)):
        assert np.array_equal(a, b), i  # deterministic
        assert rel_err(a, ref) <= TOL, (i, specs[i], rel_err(a, ref))


def test_gemv_grouped_7168_six_jobs():
    """The 7168 x 7168 workload as the benchmark runs it: FP2/FP3/FP4 x
    q = 1, 4 in one launch."""
    torch = need_gpu()
    say("gemv grouped 7168 x 6")
    specs = [(fmt, q, 7168, 7168) for fmt in FMTS for q in (1, 4)]
    for i, (a, b, ref) in enumerate(_grouped(torch, specs, seed=60, big=True)):
        err = rel_err(a, ref)
        say(f"  job {specs[i][:2]} rel err {err:.3e}")
        assert np.array_equal(a, b) and err <= TOL, i
