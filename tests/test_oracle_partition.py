"""Pins of the oracle's skew-balanced work partition.

UBEP sec. 3.3 ("Token-level Load Partition", Algorithm 1): the slots of the
send buffer are cut into equal contiguous slices, one per worker (sizes
differ by at most one), and each slice start is mapped to the expert whose
cumulative range covers it plus the offset inside that expert.

StrataCL sec. 6.2 and App. B: transfer units are assigned to cores by an
LPT-style list scheduler -- longest first, to the least-loaded core -- with
at most one unit per core per stripe and a per-peer cap on the units of one
stripe.  Without a binding cap this is Graham's LPT rule, whose makespan is
at most (4/3 - 1/(3C)) times the optimum (the bound StrataCL quotes).

Pins: the slot -> expert map built by expanding the counts, numpy's
searchsorted, Algorithm 1 run as printed (with the stop rule read as
"the window holds one expert"), Graham's tight instance, the bound against
brute-forced optima, and the cap and one-unit-per-stripe invariants.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def random_offsets(rng, E, max_count, empty_frac=0.3):
    counts = rng.integers(0, max_count + 1, size=E)
    counts[rng.random(E) < empty_frac] = 0
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def algorithm1(slot_expert, E, target):
    """UBEP Algorithm 1 (quaternary search) over the reordered expert list
    `slot_expert` (expert id of every slot, in slot order).  VectorCount(E < P)
    counts the slots whose expert is below P.  The printed loop keeps going
    while its gap is >= 1, which never ends once R - L = 1; it is read here
    as stopping when the window holds one expert."""
    def count_below(pv):
        return int(np.count_nonzero(slot_expert < pv))
    L, R, CL = 0, E, 0
    gap = math.ceil((R - L) / 4)
    while gap >= 1 and R - L > 1:
        piv = [L + i * gap for i in (1, 2, 3)]
        cnt = [count_below(pv) for pv in piv]
        P = [L] + piv + [R]
        Cs = [CL] + cnt
        q = next((i for i in (1, 2, 3) if target < cnt[i - 1]), 4)
        L, R = P[q - 1], min(P[q], R)
        CL = Cs[q - 1]
        gap = math.ceil((R - L) / 4)
        if R <= L or gap == 0:
            break
    return L, target - count_below(L)


@pytest.mark.parametrize("seed", range(12))
def test_slices_equal_sizes_and_covering_expert(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 80))
    eo = random_offsets(rng, E, 40)
    S = int(eo[-1])
    slot_expert = np.repeat(np.arange(E), np.diff(eo))
    for P in (1, 2, 3, 7, 16, 64, 100):
        start, expert, offset = oracle.slices(eo, P)
        sizes = np.diff(start)
        assert start[0] == 0 and start[-1] == S and np.all(sizes >= 0)
        assert sizes.max() - sizes.min() <= 1               # at most one slot of imbalance
        assert sizes.sum() == S
        for p in range(P):
            if start[p] == S:
                assert expert[p] == E and offset[p] == 0
                continue
            e = slot_expert[start[p]]
            assert expert[p] == e
            assert offset[p] == start[p] - eo[e]
            assert expert[p] == np.searchsorted(eo, start[p], side="right") - 1


@pytest.mark.parametrize("seed", range(8))
def test_slices_agree_with_algorithm1(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 300))
    eo = random_offsets(rng, E, 12, empty_frac=0.5)
    S = int(eo[-1])
    if S == 0:
        return
    slot_expert = np.repeat(np.arange(E), np.diff(eo))
    start, expert, offset = oracle.slices(eo, 37)
    for p in range(37):
        if start[p] < S:
            assert (expert[p], offset[p]) == algorithm1(slot_expert, E, int(start[p]))


def test_slices_skewed_hot_experts():
    # 10% of 256 experts hold half of the 131072 slots (the incast shape)
    E, S = 256, 131072
    counts = np.full(E, (S // 2) // (E - 26), np.int64)
    counts[:26] = (S // 2) // 26
    counts[-1] += S - counts.sum()
    eo = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    start, expert, offset = oracle.slices(eo, 256)
    sizes = np.diff(start)
    assert sizes.max() - sizes.min() <= 1 and sizes.sum() == S
    assert np.all(expert[:128] < 26)          # the first half of the workers serve hot experts


def makespan(load):
    return float(np.max(load)) if len(load) else 0.0


def brute_force_opt(cost, C):
    best = math.inf
    for assign in itertools.product(range(C), repeat=len(cost)):
        loads = [0.0] * C
        for j, c in enumerate(assign):
            loads[c] += cost[j]
        best = min(best, max(loads))
    return best


def test_lpt_graham_tight_instance():
    # Graham: 2C+1 jobs 2C-1, 2C-1, ..., C+1, C+1, C, C, C; LPT gives 4C-1, the
    # optimum 3C.  C = 2: jobs 3, 3, 2, 2, 2 -> 7 against 6.
    core, stripe, load = oracle.lpt([3, 3, 2, 2, 2], [0] * 5, [2], 2)
    assert makespan(load) == 7.0
    assert brute_force_opt([3, 3, 2, 2, 2], 2) == 6.0
    # C = 3: 5, 5, 4, 4, 3, 3, 3 -> 11 against 9
    cost = [5, 5, 4, 4, 3, 3, 3]
    _, _, load = oracle.lpt(cost, [0] * 7, [3], 3)
    assert makespan(load) == 11.0 and brute_force_opt(cost, 3) == 9.0


@pytest.mark.parametrize("seed", range(25))
def test_lpt_within_graham_bound(seed):
    rng = np.random.default_rng(200 + seed)
    C = int(rng.integers(2, 4))
    U = int(rng.integers(1, 8))
    cost = rng.integers(1, 20, size=U).astype(np.float64)
    peer = rng.integers(0, 3, size=U).astype(np.int32)
    cap = np.full(3, C, np.int32)                       # never binding: C cores per stripe
    core, stripe, load = oracle.lpt(cost, peer, cap, C)
    opt = brute_force_opt(list(cost), C)
    assert makespan(load) <= (4 / 3 - 1 / (3 * C)) * opt + 1e-9
    # without a binding cap no stripe is skipped: each core's stripes are 0..n-1
    for c in range(C):
        assert sorted(stripe[core == c]) == list(range(int(np.sum(core == c))))


@pytest.mark.parametrize("seed", range(10))
def test_lpt_cap_and_stripe_invariants(seed):
    rng = np.random.default_rng(300 + seed)
    C, npeer, U = 4, 5, 60
    cost = rng.integers(1, 50, size=U).astype(np.float64)
    peer = rng.integers(0, npeer, size=U).astype(np.int32)
    peer[:20] = 0                                       # a hot peer
    cap = rng.integers(1, 3, size=npeer).astype(np.int32)
    core, stripe, load = oracle.lpt(cost, peer, cap, C)
    assert np.all((core >= 0) & (core < C))
    # one unit per core per stripe
    pairs = set(zip(core.tolist(), stripe.tolist()))
    assert len(pairs) == U
    # the fan-out cap: units of one peer in one stripe
    for (k, p) in set(zip(stripe.tolist(), peer.tolist())):
        assert np.sum((stripe == k) & (peer == p)) <= cap[p]
    np.testing.assert_allclose(load, [cost[core == c].sum() for c in range(C)])


def test_lpt_equal_costs_round_robin_balance():
    core, stripe, load = oracle.lpt(np.full(23, 2.0), np.zeros(23, np.int32), [8], 8)
    assert load.max() - load.min() <= 2.0 and load.sum() == 46.0


def test_lpt_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.lpt([1.0], [3], [1, 1], 2)               # peer outside [0, npeer)
    with pytest.raises(ValueError):
        oracle.lpt([1.0], [0], [0], 2)                  # cap below one
