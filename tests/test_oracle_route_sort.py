"""Pins for the oracle's routing and align/sort (CPU only).

Routing is the plain softmax top-k with renormalisation (apply_monolithic on
the vLLM mxfp4 API page routes inside the kernel; the rule itself is the
plain reading). Pins: brute force by a full stable sort, scipy's softmax when
topk == E, weight exactly 1 when topk == 1.
"""
import numpy as np
import pytest
from scipy.special import softmax

import synth


def _brute_route(logits, topk, renorm=True):
    T, E = logits.shape
    ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :topk].astype(np.int32)
    p = softmax(logits.astype(np.float64), axis=1)
    w = np.take_along_axis(p, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


@pytest.mark.parametrize("T,E,topk", [(4, 8, 2), (7, 16, 5), (3, 112, 15), (5, 6, 6), (9, 10, 1)])
def test_route_brute_force(orc, T, E, topk):
    rng = np.random.default_rng(T * 100 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route_topk(logits, topk)
    bids, bw = _brute_route(logits, topk)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=2e-7, atol=1e-9)


def test_route_ties_go_to_lower_index(orc):
    logits = np.array([[1, 3, 3, 0, 3, 2], [0, 0, 0, 0, 0, 0]], dtype=np.float32)
    ids, w = orc.route_topk(logits, 4)
    assert ids.tolist() == [[1, 2, 4, 5], [0, 1, 2, 3]]
    np.testing.assert_allclose(w[1], [0.25] * 4, rtol=1e-7)


def test_route_topk_equals_E_is_full_softmax(orc):
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((6, 12)) * 4).astype(np.float32)
    ids, w = orc.route_topk(logits, 12)
    full = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, axis=1), rtol=2e-7)
    assert np.all(np.diff(np.take_along_axis(logits, ids, axis=1), axis=1) <= 0)


def test_route_topk1_weight_is_one(orc):
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((10, 20)).astype(np.float32)
    ids, w = orc.route_topk(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_route_without_renormalisation(orc):
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((5, 9)).astype(np.float32)
    ids, w = orc.route_topk(logits, 3, renormalize=False)
    bids, bw = _brute_route(logits, 3, renorm=False)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=2e-7)
    assert np.all(w.sum(axis=1) < 1.0)


def test_route_production_invariants(orc):
    wl = synth.make(synth.specs()["skewed_t32"], with_weights=False)
    ids, w = orc.route_topk(wl.logits, 15)
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == 15
        assert np.all(np.diff(wl.logits[t, ids[t]]) <= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    # the hot experts receive most of the traffic
    hot = set(wl.hot_experts.tolist())
    frac = np.mean([e in hot for e in ids.ravel()])
    assert frac > 8 * 32 / ids.size * 0.9


def _brute_sort(ids, E, bm):
    P = ids.size
    flat = ids.ravel()
    order = sorted(range(P), key=lambda p: (flat[p], p))
    out, be, off = [], [], []
    i = 0
    for e in range(E):
        off.append(len(out))
        seg = [p for p in order if flat[p] == e]
        if seg:
            pad = (len(seg) + bm - 1) // bm * bm
            seg = seg + [P] * (pad - len(seg))
            out += seg
            be += [e] * (pad // bm)
    off.append(len(out))
    return out, be, off


@pytest.mark.parametrize("T,E,topk,bm", [(4, 8, 2, 16), (1, 112, 15, 16), (32, 112, 15, 32),
                                         (7, 16, 3, 64), (50, 8, 4, 16), (0, 8, 2, 16)])
def test_align_sort_brute_force(orc, T, E, topk, bm):
    rng = np.random.default_rng(T + E)
    rows = [rng.permutation(E)[:topk] for _ in range(T)]
    ids = (np.stack(rows) if rows else np.zeros((0, topk))).astype(np.int32).reshape(T, topk)
    sorted_ids, be, off, npp = orc.align_sort(ids, E, bm)
    bsorted, bbe, boff = _brute_sort(ids, E, bm)
    cap = orc.align_capacity(T, topk, E, bm)
    assert cap % bm == 0 and cap >= len(bsorted)
    assert npp == len(bsorted)
    assert sorted_ids[:npp].tolist() == bsorted
    assert np.all(sorted_ids[npp:] == T * topk)
    assert be[:npp // bm].tolist() == bbe
    assert np.all(be[npp // bm:] == -1)
    assert off.tolist() == boff
    real = sorted_ids[sorted_ids < T * topk]
    assert sorted(real.tolist()) == list(range(T * topk))


def test_align_sort_skewed_segments(orc):
    wl = synth.make(synth.specs()["skewed_t16"], with_weights=False)
    ids, _ = orc.route_topk(wl.logits, 15)
    bm = 16
    sorted_ids, be, off, npp = orc.align_sort(ids, 112, bm)
    hist = np.bincount(ids.ravel(), minlength=112)
    for e in range(112):
        seg = sorted_ids[off[e]:off[e + 1]]
        real = seg[seg < ids.size]
        assert len(real) == hist[e]
        assert np.all(np.diff(real) > 0)
        assert np.all(ids.ravel()[real] == e)
        assert len(seg) == (hist[e] + bm - 1) // bm * bm
