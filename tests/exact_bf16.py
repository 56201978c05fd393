"""Exact rational statements of the bf16 format and of round-to-nearest-even,
written from the format's definition (1 sign bit, 8 exponent bits with bias
127, 7 fraction bits; subnormals below 2^-126).  Used by the oracle pins as a
check that shares nothing with the oracle's own C rounding."""
import math
from fractions import Fraction

import numpy as np

from combine_ep_route_topk_amd import workloads as wl


def bf16_exact(b):
    """Exact value of a finite bf16 pattern as a Fraction, from the format."""
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def rne_bf16_exact(v: Fraction, negative_zero=False):
    """Round an exact rational to bf16 (nearest, ties to even) -> pattern."""
    if v == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent of the leading bit
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)                    # quantum exponent
    n = a / Fraction(2) ** q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * Fraction(2) ** q
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    if r < Fraction(2) ** -126:
        return sign | int(r / Fraction(2) ** -133)
    e2 = e if r < Fraction(2) ** (e + 1) else e + 1
    frac = int((r / Fraction(2) ** e2 - 1) * 128)
    return sign | ((e2 + 127) << 7) | frac


def f32_tie_products(n, seed):
    """(w f32, g bf16 bits) pairs whose exact product is NOT a bf16 tie but
    whose f32 rounding IS one, on the side where ties-to-even goes the other
    way: a product first rounded to f32 and then to bf16 comes out one bf16
    step off on these."""
    rng = np.random.default_rng(seed)
    ws, gs = [], []
    while len(ws) < n:
        g_bits = int(wl.f32_to_bf16_bits(np.array([rng.uniform(1.0, 2.0)], np.float32))[0]) | 0x1
        g = float(wl.bf16_bits_to_f32(np.array([g_bits], np.uint16))[0])
        below = int(rng.integers(0x3F80, 0x4000))      # bf16 pattern in [1, 2)
        target = float(np.array([(below << 16) | 0x8000], np.uint32).view(np.float32)[0])
        w = np.float32(target / g)
        exact = float(w) * g                           # exact: 24 x 8 bits
        even_goes_down = below % 2 == 0
        if float(np.float32(exact)) == target and (exact > target) == even_goes_down:
            ws.append(w)
            gs.append(g_bits)
    return np.array(ws, np.float32), np.array(gs, np.uint16)


def plant_tie_products(w, g_bits, tokens, seed):
    """Puts one f32_tie_products pair at pick 0, column 0 of each listed token:
    w[t][0] and g[t][0] change in place."""
    ws, gs = f32_tie_products(len(tokens), seed)
    for i, t in enumerate(tokens):
        w[t, 0] = ws[i]
        g_bits[t, 0] = gs[i]


# ---------------------------------------------------------------- binary32
# IEEE 754 binary32: 24 significant bits, exponents -126..127, subnormals with
# quantum 2^-149.  Finite values are carried as a Fraction plus a flag for -0;
# a rounding that overflows gives the float infinities.

F32_MAX_EXP = 127
F32_MIN_QUANTUM = -149


def rne_f32_exact(v: Fraction):
    """Round an exact rational to binary32, nearest, ties to even.  Returns
    the rounded value as a Fraction, or +-math.inf on overflow (a result whose
    rounding with an unbounded exponent reaches 2^128)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, F32_MIN_QUANTUM)
    n = a / Fraction(2) ** q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * Fraction(2) ** q
    if r >= Fraction(2) ** (F32_MAX_EXP + 1):
        return math.inf if v > 0 else -math.inf
    return r if v > 0 else -r


def f32_bits_exact(bits: int) -> Fraction:
    """Exact value of a finite binary32 pattern, from the format."""
    sign = -1 if bits & 0x80000000 else 1
    e = (bits >> 23) & 0xFF
    f = bits & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 1 << 23) * Fraction(2) ** -126
    return sign * (1 + Fraction(f, 1 << 23)) * Fraction(2) ** (e - 127)


def chain_combine_exact(ws, ys):
    """The combine contract on one output element, in exact arithmetic with an
    explicit binary32 rounding after every operation: acc = fl(w0 * y0), then
    acc = fl(wj * yj + acc) for j >= 1 (a fused multiply-add: the product is
    not rounded on its own), then round to bf16.  ws: binary32 patterns of the
    weights; ys: bf16 patterns.  Returns the bf16 pattern.

    Signed zeros follow IEEE 754: a product of zeros takes the xor of the
    signs; an exact sum of zero is -0 only when both addends are -0
    (round-to-nearest); a nonzero value that underflows to zero keeps its
    sign.  The addends are finite, so an accumulator that overflowed to an
    infinity stays that infinity."""
    acc, acc_neg0 = None, False
    for j, (wb, yb) in enumerate(zip(ws, ys)):
        w = f32_bits_exact(wb)
        y = bf16_exact(yb)
        prod_neg = bool(wb & 0x80000000) != bool(yb & 0x8000)
        p = w * y
        if j == 0:
            if p == 0:
                acc, acc_neg0 = Fraction(0), prod_neg
            else:
                acc = rne_f32_exact(p)
                acc_neg0 = acc == 0 and p < 0
            continue
        if isinstance(acc, float):          # an infinity: stays (finite addends)
            continue
        s = p + acc
        if s == 0:
            both_neg0 = (p == 0 and prod_neg) and (acc == 0 and acc_neg0)
            acc, acc_neg0 = Fraction(0), both_neg0
        else:
            acc = rne_f32_exact(s)
            acc_neg0 = acc == 0 and s < 0
    if isinstance(acc, float):
        return 0x7F80 if acc > 0 else 0xFF80
    return rne_bf16_exact(acc, negative_zero=acc_neg0)
