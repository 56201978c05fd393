"""Pins of the oracle's router (top-k selection + softmax gating).

The oracle is pinned to things other than itself: hand-derived fixtures,
brute force by a full stable sort, scipy's softmax, closed forms and the
invariants of a probability vector.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_route_cases():
    with open(os.path.join(GOLDEN, "route_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        logits = np.array(c["logits"], np.float32)
        idx, w = oracle.route_topk(logits, c["k"], c["normalize"])
        assert idx.tolist() == c["idx"], c
        np.testing.assert_allclose(w.astype(np.float64), np.array(c["w"]),
                                   rtol=0, atol=c["w_tol"] + 1e-12)


def brute_topk(logits, k):
    # full stable sort by descending logit: ties keep the lower index first
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 1), (33, 256, 8, 2), (50, 128, 8, 3),
                                        (20, 5, 5, 4), (17, 64, 1, 5)])
def test_topk_matches_full_sort(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    # plant ties: copy some logits onto other experts of the same token
    logits[:, E // 2] = logits[:, 0]
    idx, w = oracle.route_topk(logits, k, 1)
    np.testing.assert_array_equal(idx, brute_topk(logits, k))
    # picks are distinct, in range, and no unpicked expert beats the last pick
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
        last = logits[t, idx[t, -1]]
        rest = np.setdiff1d(np.arange(E), idx[t])
        assert np.all((logits[t, rest] < last) |
                      ((logits[t, rest] == last) & (rest > idx[t, -1])))


def test_ties_with_signed_zero_and_quantized_logits():
    rng = np.random.default_rng(7)
    logits = rng.integers(-3, 4, size=(200, 16)).astype(np.float32) * np.float32(0.5)
    logits[logits == 0] = np.where(rng.random((logits == 0).sum()) < 0.5, -0.0, 0.0)
    idx, _ = oracle.route_topk(logits, 6, 1)
    np.testing.assert_array_equal(idx, brute_topk(logits, 6))


@pytest.mark.parametrize("normalize", [0, 1])
def test_weights_vs_scipy_softmax(normalize):
    rng = np.random.default_rng(11)
    T, E, k = 40, 256, 8
    logits = rng.standard_normal((T, E), dtype=np.float32) * np.float32(3)
    idx, w = oracle.route_topk(logits, k, normalize)
    for t in range(T):
        lt = logits[t].astype(np.float64)
        ref = softmax(lt[idx[t]]) if normalize else softmax(lt)[idx[t]]
        # the oracle's only error is the final rounding to f32
        np.testing.assert_allclose(w[t].astype(np.float64), ref, rtol=2 ** -24, atol=0)
    if normalize:
        np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=k * 2 ** -24)
    else:
        assert np.all(w.astype(np.float64).sum(1) <= 1.0 + k * 2 ** -24)
    # weights follow the pick order
    assert np.all(np.diff(w, axis=1) <= 0)


def test_special_cases():
    # all logits equal: picks 0..k-1, uniform weights
    idx, w = oracle.route_topk(np.full((3, 8), 0.25, np.float32), 4, 1)
    assert idx.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == np.float32(0.25))
    # k == E: normalize=0 and normalize=1 coincide
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((10, 6), dtype=np.float32)
    i0, w0 = oracle.route_topk(lg, 6, 0)
    i1, w1 = oracle.route_topk(lg, 6, 1)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_allclose(w0, w1, rtol=2 ** -23)
    # k == 1, normalize=1: the single weight is exactly 1
    _, w = oracle.route_topk(lg, 1, 1)
    assert np.all(w == 1.0)


def test_rejects_non_finite():
    lg = np.zeros((2, 4), np.float32)
    lg[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route_topk(lg, 2, 1)
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((2, 4), np.float32), 5, 1)
