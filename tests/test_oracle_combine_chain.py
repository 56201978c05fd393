"""Pins of the oracle's combine contract: fp32 accumulation in the fixed top-k
order (HyperParallel-MoE sec. 4.1: Combine accumulates the top-k expert
contributions by routing score).  For each output element

    acc = fl32(w0 * y0);  acc = fl32(wj * yj + acc) for j = 1..k-1;  bf16_rne(acc)

with fl32 one IEEE binary32 rounding (the later steps are fused multiply-adds).

The oracle's C code is pinned to things other than itself:
  - hand-derived bit patterns (tests/golden/combine_chain.json), each case
    built so that one plausible mistake changes its output: rounding the
    product before the add, summing in higher precision, reordering the
    picks, starting from a +0 accumulator, missing an fp32 overflow, and
    subnormal rounding;
  - exact rational arithmetic with an explicit binary32 rounding after every
    operation (tests/exact_bf16.py, written from the format), on random and
    on adversarial inputs with heavy cancellation;
  - the exact weighted sum (combine_exact, pinned in
    test_oracle_dispatch_combine.py) within the derived error bound of k fp32
    roundings;
  - cases where every fp32 step is exact, on which the chain must equal the
    exact sum bit for bit;
  - the identities: a weight-1 top-1 combine is a gather, one-hot weights
    select a row, combine(dispatch(x)) == x with normalized routing weights.
dispatch_grad (a unit-weight sum in pick order) is pinned the same way.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_ep_route_topk_amd import workloads as wl
from exact_bf16 import chain_combine_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE_BITS = 0x3F800000


def _golden():
    with open(os.path.join(GOLDEN, "combine_chain.json")) as f:
        return json.load(f)["cases"]


def _weights(c):
    return np.array(c["w_bits"], np.uint32).view(np.float32)


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_chain_cases(case):
    y = np.array(case["y"], np.uint16)
    pos = np.array(case["pos"], np.int32)
    w = _weights(case)
    assert oracle.combine(y, pos, w).reshape(-1).tolist() == case["out"], case["why"]
    assert oracle.combine_exact(y, pos, w).reshape(-1).tolist() == case["exact_out"], case["why"]
    # the rational evaluator agrees with the hand derivation too
    for t in range(case["T"]):
        ws = [int(b) for b in np.array(case["w_bits"][t], np.uint32)]
        ys = [int(y[pos[t, j], 0]) for j in range(case["k"])]
        assert chain_combine_exact(ws, ys) == case["out"][t], case["why"]


def test_golden_small_cases_hold_for_the_chain():
    # every case of combine_small.json is exact at every fp32 step, so the
    # chain and the exact sum give the same hand-derived patterns
    with open(os.path.join(GOLDEN, "combine_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        args = (np.array(c["y"], np.uint16), np.array(c["pos"], np.int32),
                np.array(c["w"], np.float32))
        assert oracle.combine(*args).reshape(-1).tolist() == c["out"], c["why"]


def _rational_check(y, pos, w):
    out = oracle.combine(y, pos, w)
    wb = w.view(np.uint32)
    T, k = pos.shape
    for t in range(T):
        for h in range(y.shape[1]):
            ref = chain_combine_exact([int(b) for b in wb[t]],
                                      [int(y[pos[t, j], h]) for j in range(k)])
            assert out[t, h] == ref, (t, h, hex(int(out[t, h])), hex(ref))
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])
def test_chain_vs_exact_rationals_random(k):
    rng = np.random.default_rng(300 + k)
    T, H = 12, 16
    y = wl.make_rows(T * k, H, seed=310 + k)
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w = (rng.random((T, k), dtype=np.float32) - np.float32(0.3))
    _rational_check(y, pos, w)


def _cancelling_case(seed, T, H, k):
    """Rows spread over 2^-20..2^20 whose picks cancel: pick j > 0 repeats
    pick 0 (or a previous pick) with its sign flipped about half of the time,
    under weights within a few f32 steps of +-1, so the surviving difference
    is of the order of one fp32 rounding of the products."""
    rng = np.random.default_rng(seed)
    mag = rng.standard_normal((T * k, H)) * 2.0 ** rng.integers(-20, 21, size=(T * k, H))
    y = wl.f32_to_bf16_bits(mag.astype(np.float32))
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    for t in range(T):
        for j in range(1, k):
            if rng.random() < 0.5:
                src = pos[t, int(rng.integers(0, j))]
                y[pos[t, j]] = y[src] ^ np.uint16(0x8000)
    w = (np.float32(1) + (rng.random((T, k), dtype=np.float32) - np.float32(0.5))
         * np.float32(2.0 ** -20)) * rng.choice(np.array([-1, 1], np.float32), size=(T, k))
    return y, pos, w.astype(np.float32)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_chain_vs_exact_rationals_under_cancellation(k):
    y, pos, w = _cancelling_case(400 + k, 48, 16, k)
    out = _rational_check(y, pos, w)
    # the case really does separate the chain from a single rounding of the
    # exact sum, so the check above sees the fp32 steps
    assert np.sum(out != oracle.combine_exact(y, pos, w)) > 0


def test_chain_within_the_bound_of_the_exact_sum():
    # k fp32 roundings: |acc - S| <= g_k * sum_j |w_j y_j|, g_k = k u / (1 - k u),
    # u = 2^-24; both sides then round to bf16 (half an ulp each)
    T, H, k = 256, 64, 8
    y, pos, w = _cancelling_case(501, T, H, k)
    chain = wl.bf16_bits_to_f32(oracle.combine(y, pos, w)).astype(np.float64)
    exact = wl.bf16_bits_to_f32(oracle.combine_exact(y, pos, w)).astype(np.float64)
    Y = wl.bf16_bits_to_f32(y[pos.reshape(-1)]).astype(np.float64).reshape(T, k, H)
    mag = np.einsum("tk,tkh->th", np.abs(w.astype(np.float64)), np.abs(Y))
    gam = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    a = np.maximum(np.abs(chain), np.abs(exact))
    ulp = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(a, 2.0 ** -126))), -126) - 7)
    assert np.all(np.abs(chain - exact) <= ulp + gam * mag)


def test_chain_equals_exact_sum_when_every_step_is_exact():
    # small integers times dyadic weights: every product and partial sum is
    # an f32 and every result a bf16, so no step rounds
    rng = np.random.default_rng(600)
    T, H, k = 64, 24, 8
    y = wl.f32_to_bf16_bits(rng.integers(-8, 9, size=(T * k, H)).astype(np.float32))
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w = (rng.integers(-4, 5, size=(T, k)) / 4).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine(y, pos, w), oracle.combine_exact(y, pos, w))


def test_chain_top1_weight1_is_gather_and_one_hot_selects():
    T, H, k = 16, 24, 4
    y = wl.make_rows(T * k, H, seed=701)
    pos = np.random.default_rng(702).permutation(T * k).astype(np.int32).reshape(T, k)
    perm = np.random.default_rng(703).permutation(T).astype(np.int32).reshape(T, 1)
    np.testing.assert_array_equal(oracle.combine(y[:T], perm, np.ones((T, 1), np.float32)),
                                  y[:T][perm[:, 0]])
    for hot in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, hot] = 1
        np.testing.assert_array_equal(oracle.combine(y, pos, w), y[pos[:, hot]])


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_chain_round_trip_identity_experts(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    idx, wt = oracle.route_topk(inp["logits"], w.k, 1)
    lay = oracle.dispatch_layout(idx, w.E, w.R)
    send = oracle.dispatch(inp["x"], lay["pos"])
    np.testing.assert_array_equal(oracle.combine(send, lay["pos"], wt), inp["x"])


def test_chain_tokens_match_full():
    T, H, k = 20, 16, 3
    y, pos, w = _cancelling_case(800, T, H, k)
    toks = np.array([19, 0, 7, 7], np.int64)
    np.testing.assert_array_equal(oracle.combine_tokens(y, pos, w, toks),
                                  oracle.combine(y, pos, w)[toks])


@pytest.mark.parametrize("k", [1, 3, 8])
def test_dispatch_grad_vs_exact_rationals(k):
    # grad_x = the sum of the k gradient rows in fp32, pick order: the chain
    # with unit weights (every product 1 * y is exact)
    y, pos, _ = _cancelling_case(900 + k, 12, 16, k)
    got = oracle.dispatch_grad(y, pos)
    for t in range(pos.shape[0]):
        for h in range(y.shape[1]):
            ref = chain_combine_exact([ONE_BITS] * k, [int(y[pos[t, j], h]) for j in range(k)])
            assert got[t, h] == ref, (t, h)
    np.testing.assert_array_equal(got, oracle.combine(y, pos, np.ones(pos.shape, np.float32)))
    # and the exact reference rounds the double sum once
    exact = oracle.dispatch_grad_exact(y, pos)
    np.testing.assert_array_equal(exact, oracle.combine_exact(y, pos,
                                                              np.ones(pos.shape, np.float32)))


def test_rational_evaluator_catches_planted_mistakes():
    """The evaluator and fixtures separate the chain from its plausible
    misreadings: each emulated mistake disagrees with the evaluator on at
    least one golden case."""
    from fractions import Fraction
    from exact_bf16 import bf16_exact, f32_bits_exact, rne_bf16_exact, rne_f32_exact

    def mul_then_add(ws, ys):
        acc = None
        for wb, yb in zip(ws, ys):
            p = rne_f32_exact(f32_bits_exact(wb) * bf16_exact(yb))
            acc = p if acc is None else rne_f32_exact(acc + p)
        return rne_bf16_exact(acc)

    def exact_sum(ws, ys):
        s = sum(f32_bits_exact(wb) * bf16_exact(yb) for wb, yb in zip(ws, ys))
        return rne_bf16_exact(Fraction(s))

    def reversed_order(ws, ys):
        return chain_combine_exact(ws[::-1], ys[::-1])

    for mistake in (mul_then_add, exact_sum, reversed_order):
        caught = False
        for c in _golden():
            if c["name"] in ("f32_overflow_in_the_chain", "negative_zero_first_product",
                             "opposite_zeros_sum_to_plus_zero"):
                continue                      # the emulations skip inf and -0
            y = np.array(c["y"], np.uint16)
            pos = np.array(c["pos"], np.int32)
            for t in range(c["T"]):
                ws = [int(b) for b in np.array(c["w_bits"][t], np.uint32)]
                ys = [int(y[pos[t, j], 0]) for j in range(c["k"])]
                if mistake(ws, ys) != c["out"][t]:
                    caught = True
        assert caught, mistake.__name__
