"""Pins for the oracle's router, bucketing, SwiGLU FFN and combine:
brute force over all k-subsets, constructed exact ties, softmax identities,
stable-sort properties, and the one-expert case that reduces to a dense
FFN computed with numpy from dequantized matrices."""

import itertools

import numpy as np
import pytest

import inputgen
import oracle as O


def test_topk_brute_force_all_subsets():
    rng = np.random.default_rng(0)
    for trial in range(60):
        E = int(rng.integers(5, 13))
        k = int(rng.integers(1, 5))
        H = 64
        x = rng.standard_normal((2, H)).astype(np.float32)
        Wr = rng.standard_normal((E, H)).astype(np.float32)
        r = O.route(x, Wr, None, k)
        for t in range(2):
            l = r["logits"][t]
            best = max(itertools.combinations(range(E), k), key=lambda s: sum(l[list(s)]))
            assert sorted(best) == sorted(r["idx"][t].tolist())
            # order inside the top-k: descending logit
            assert np.all(np.diff(l[r["idx"][t]]) <= 0)


def test_topk_exact_ties_go_to_lower_id():
    E, H = 8, 32
    Wr = np.zeros((E, H), np.float32)
    for e in range(E):
        Wr[e, 0] = [1, 3, 3, 2, 3, 0, 2, 1][e]
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    r = O.route(x, Wr, None, 5)
    assert r["idx"][0].tolist() == [1, 2, 4, 3, 6]


def test_bias_enters_selection_and_weights():
    E, H = 6, 16
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, H)).astype(np.float32)
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    b = np.array([0, 0, 50, 0, 0, 0], np.float32)
    r = O.route(x, Wr, b, 2)
    assert np.all(r["idx"][:, 0] == 2)
    rb = O.route(x, Wr, None, 2)
    assert np.allclose(r["logits"], rb["logits"] + b[None, :].astype(np.float64))


def test_softmax_identities():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    Wr = (rng.standard_normal((256, 128)) * 0.1).astype(np.float32)
    r = O.route(x, Wr, None, 6)
    p, l = r["probs"], r["logits"]
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    for t in range(4):
        i, j = r["idx"][t][0], r["idx"][t][5]
        assert p[t, i] / p[t, j] == pytest.approx(np.exp(l[t, i] - l[t, j]), rel=1e-12)
    assert np.array_equal(r["w"], np.take_along_axis(p, r["idx"].astype(np.int64), 1))
    # weights are not renormalised
    assert np.all(r["w"].sum(1) < 1.0)


def test_bucket_is_a_stable_grouping():
    rng = np.random.default_rng(4)
    for trial in range(50):
        T, k, E = int(rng.integers(1, 40)), int(rng.integers(1, 7)), int(rng.integers(6, 300))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        ps, off = O.bucket(idx, E)
        flat = idx.reshape(-1)
        assert sorted(ps.tolist()) == list(range(T * k))
        ids = flat[ps]
        assert np.all(np.diff(ids) >= 0)
        for e in range(E):
            seg = ps[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e)
            assert np.all(np.diff(seg) > 0)  # stable: pair order kept
        assert off[0] == 0 and off[-1] == T * k


def test_silu_values():
    assert O.silu(0.0) == 0.0
    assert O.silu(50.0) == pytest.approx(50.0)
    assert O.silu(-50.0) == pytest.approx(0.0, abs=1e-19)
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)))


def test_one_expert_reduces_to_dense_ffn():
    """E = 1, k = 1: the MoE FFN is a dense SwiGLU FFN; compare with numpy
    fp64 products of the dequantized matrices (h requantized by the
    separately pinned activation quantizer)."""
    H, I = 128, 64
    G = inputgen.expert_weight(0, 0, inputgen.MAT_GATE, I, H)
    U = inputgen.expert_weight(0, 0, inputgen.MAT_UP, I, H)
    D = inputgen.expert_weight(0, 0, inputgen.MAT_DOWN, H, I)
    gb, ub, db = O.quantize_matrix(2, G), O.quantize_matrix(2, U), O.quantize_matrix(3, D)
    x = inputgen.tokens(0, 0, 2, H)
    xq, xs = O.quantize_act(x)
    res = O.ffn(2, gb, 2, ub, 3, db, xq, xs)
    xd = xq * np.repeat(xs.astype(np.float64), 32, 1)
    g = xd @ O.dequantize_matrix(2, gb).T
    u = xd @ O.dequantize_matrix(2, ub).T
    assert np.allclose(res["g"], g, rtol=1e-12, atol=1e-15)
    assert np.allclose(res["u"], u, rtol=1e-12, atol=1e-15)
    h = g / (1 + np.exp(-g)) * u
    hq, hs = O.quantize_act(h.astype(np.float32))
    assert np.array_equal(hq, res["hq"])
    hd = hq * np.repeat(hs.astype(np.float64), 32, 1)
    o = hd @ O.dequantize_matrix(3, db).T
    assert np.allclose(res["o"], o, rtol=1e-12, atol=1e-15)


def test_combine_order_and_values():
    rng = np.random.default_rng(5)
    osh = rng.standard_normal((3, 10))
    op = rng.standard_normal((3, 4, 10))
    w = rng.uniform(0, 1, (3, 4))
    y = O.combine(osh, op, w)
    assert np.allclose(y, osh + np.einsum("tj,tjh->th", w, op), rtol=1e-14)
