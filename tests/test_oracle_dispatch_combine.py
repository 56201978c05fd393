"""Pins of the oracle's dispatch copy, exact combine reduction and bf16 rounding.

combine_exact (the one rounding of the exact weighted sum, the accuracy
reference for the fp32 combine chain pinned in test_oracle_combine_chain.py)
is pinned against hand-derived bit patterns, exact rational arithmetic
(fractions.Fraction) for the weighted sum and its round-to-nearest-even,
an independent bit-level f32 -> bf16 rounding, and the identities of the
method: a weight-1 top-1 combine is a gather, one-hot weights select a row,
and combine(dispatch(x)) with weights summing to one returns x exactly.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from combine_ep_route_topk_amd import workloads as wl
from exact_bf16 import bf16_exact, rne_bf16_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 pins

def test_bf16_to_double_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        ref = wl.bf16_bits_to_f32(pats).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_double_to_bf16_hand_values():
    cases = [  # (value, expected pattern); a list, since -0.0 == 0.0 as dict keys
        (1.0, 0x3F80), (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82),
        (1.0 + 2 ** -8 + 2 ** -40, 0x3F81), (-2.5, 0xC020), (2.0 ** -133, 0x0001),
        (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002), (2.0 ** -126, 0x0080),
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F), ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),
        ((2 - 2 ** -8 - 2 ** -30) * 2.0 ** 127, 0x7F7F), (-0.0, 0x8000), (0.0, 0x0000),
        (math.inf, 0x7F80), (-math.inf, 0xFF80),
    ]
    for v, b in cases:
        assert oracle.double_to_bf16(v) == b, (v, hex(oracle.double_to_bf16(v)), hex(b))
    assert oracle.double_to_bf16(math.nan) & 0x7FC0 == 0x7FC0


def test_double_to_bf16_vs_bit_rounding_of_f32():
    # values exactly representable in f32: the double path must agree with the
    # independent integer rounding of the f32 bit pattern
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = wl.f32_to_bf16_bits(f)
    got = np.array([oracle.double_to_bf16(float(v)) for v in f], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_double_to_bf16_vs_exact_rationals():
    rng = np.random.default_rng(6)
    for _ in range(3000):
        v = float(rng.standard_normal()) * 2.0 ** int(rng.integers(-140, 130))
        assert oracle.double_to_bf16(v) == rne_bf16_exact(Fraction(v),
                                                          negative_zero=math.copysign(1, v) < 0)


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_dispatch_places_every_row(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    idx, _ = oracle.route_topk(inp["logits"], w.k, 1)
    lay = oracle.dispatch_layout(idx, w.E, w.R)
    send = np.full((w.S, w.H), 0xFFFF, np.uint16)      # poison
    oracle.dispatch(inp["x"], lay["pos"], out=send)
    assert not np.any(np.all(send == 0xFFFF, axis=1))  # every slot written
    for t in range(w.T):
        for j in range(w.k):
            np.testing.assert_array_equal(send[lay["pos"][t, j]], inp["x"][t])
    # slot_src names the token that fills each slot
    np.testing.assert_array_equal(send, inp["x"][lay["slot_src"] // w.k])


# ---------------------------------------------------------------- combine

def test_golden_combine_cases():
    with open(os.path.join(GOLDEN, "combine_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        out = oracle.combine_exact(np.array(c["y"], np.uint16), np.array(c["pos"], np.int32),
                                   np.array(c["w"], np.float32))
        assert out.reshape(-1).tolist() == c["out"], c["why"]


def test_combine_vs_exact_rationals():
    rng = np.random.default_rng(8)
    T, H, k = 6, 24, 8
    y = wl.make_rows(T * k, H, seed=9)
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w = (rng.random((T, k), dtype=np.float32) - np.float32(0.3))
    out = oracle.combine_exact(y, pos, w)
    for t in range(T):
        for h in range(H):
            exact = sum(Fraction(float(w[t, j])) * bf16_exact(int(y[pos[t, j], h]))
                        for j in range(k))
            assert out[t, h] == rne_bf16_exact(exact), (t, h)


def test_combine_top1_weight1_is_gather():
    T, H = 32, 40
    y = wl.make_rows(T, H, seed=12)
    pos = np.random.default_rng(1).permutation(T).astype(np.int32).reshape(T, 1)
    out = oracle.combine_exact(y, pos, np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(out, y[pos[:, 0]])


def test_combine_one_hot_selects_row():
    T, H, k = 16, 24, 4
    y = wl.make_rows(T * k, H, seed=13)
    pos = np.arange(T * k, dtype=np.int32).reshape(T, k)
    for hot in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, hot] = 1
        np.testing.assert_array_equal(oracle.combine_exact(y, pos, w), y[pos[:, hot]])


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_round_trip_identity_experts(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    idx, wt = oracle.route_topk(inp["logits"], w.k, 1)
    lay = oracle.dispatch_layout(idx, w.E, w.R)
    send = oracle.dispatch(inp["x"], lay["pos"])
    out = oracle.combine_exact(send, lay["pos"], wt)
    np.testing.assert_array_equal(out, inp["x"])


def test_combine_sampled_tokens_match_full():
    T, H, k = 20, 16, 3
    y = wl.make_rows(T * k, H, seed=14)
    pos = np.random.default_rng(2).permutation(T * k).astype(np.int32).reshape(T, k)
    w = np.random.default_rng(3).random((T, k), dtype=np.float32)
    full = oracle.combine(y, pos, w)
    toks = np.array([19, 0, 7, 7], np.int64)
    np.testing.assert_array_equal(oracle.combine_tokens(y, pos, w, toks), full[toks])


def test_fused_trailer_layout():
    tr = oracle.fused_trailers(0x0123456789ABCDEF, np.array([5, 70000], np.int32))
    assert bytes(tr[0]) == bytes.fromhex("efcdab8967452301" "05000000" "00000000")
    assert bytes(tr[1]) == bytes.fromhex("efcdab8967452301" "70110100" "00000000")
