"""The library's host-side LPT scheduler (ep_lpt_partition; StrataCL sec. 6.2,
App. B) against the oracle's, on the CPU: the same units, cores, stripes and
loads, bit for bit, on uniform, skewed and multi-tier inputs."""
import ctypes

import numpy as np
import pytest

import oracle


class Task(ctypes.Structure):
    _fields_ = [("peer", ctypes.c_int32), ("stripe", ctypes.c_int32),
                ("first_row", ctypes.c_int64), ("rows", ctypes.c_int64), ("cost", ctypes.c_double)]


@pytest.fixture(scope="module")
def lib():
    from combine_ep_route_topk_amd import ep
    L = ep.library()
    P = ctypes.c_void_p
    L.ep_lpt_task_count.argtypes = [P, ctypes.c_int32, ctypes.c_int64]
    L.ep_lpt_task_count.restype = ctypes.c_int64
    L.ep_lpt_partition.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, P, P, P,
                                   ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P, P]
    L.ep_lpt_partition.restype = ctypes.c_int
    return L


def p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def units(ro, row_bytes, unit_rows, tier, alpha, beta):
    """The transfer units StrataCL describes: each peer window in pieces of
    unit_rows rows, cost alpha_t + bytes / beta_t (peer-major, row order)."""
    cost, peer, first, rows = [], [], [], []
    for q in range(len(ro) - 1):
        t = 0 if tier is None else tier[q]
        for r in range(ro[q], ro[q + 1], unit_rows):
            n = min(unit_rows, ro[q + 1] - r)
            cost.append(alpha[t] + float(n * row_bytes) / beta[t])
            peer.append(q)
            first.append(r)
            rows.append(n)
    return (np.array(cost, np.float64), np.array(peer, np.int32), np.array(first, np.int64),
            np.array(rows, np.int64))


def run_lib(L, ro, row_bytes, unit_rows, tier, alpha, beta, cap, C):
    R = len(ro) - 1
    n = L.ep_lpt_task_count(p(ro), R, unit_rows)
    tasks = (Task * max(n, 1))()
    core_begin = np.zeros(C + 1, np.int64)
    load = np.zeros(C, np.float64)
    rc = L.ep_lpt_partition(p(ro), R, row_bytes, unit_rows, p(tier), p(alpha), p(beta), p(cap),
                            len(alpha), C, ctypes.cast(tasks, ctypes.c_void_p), n, p(core_begin),
                            p(load))
    assert rc == 0, L.ep_last_error().decode()
    return tasks, n, core_begin, load


CASES = [
    # R, rows per peer (generator), unit_rows, C, tiers
    (8, "uniform", 64, 4, 1),
    (32, "skewed", 128, 16, 1),
    (64, "skewed", 256, 64, 1),
    (16, "random", 50, 7, 2),
    (5, "random", 1000, 12, 3),      # more cores than units
    (64, "incast", 512, 256, 1),
]


@pytest.mark.parametrize("R,kind,unit_rows,C,ntier", CASES)
def test_lpt_partition_matches_oracle(lib, R, kind, unit_rows, C, ntier):
    rng = np.random.default_rng(R * 31 + C)
    if kind == "uniform":
        counts = np.full(R, 512)
    elif kind == "skewed":
        counts = (rng.zipf(1.2, size=R) * 97) % 5000
    elif kind == "incast":
        counts = np.full(R, 1024)
        counts[: max(1, R // 10)] = 16 * 1024
    else:
        counts = rng.integers(0, 3000, size=R)
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_bytes = 14336
    tier = None if ntier == 1 else rng.integers(0, ntier, size=R).astype(np.int32)
    alpha = np.array([2000.0, 3500.0, 9000.0][:ntier])
    beta = np.array([100.0, 60.0, 30.0][:ntier])
    cap = np.array([max(1, C // 4), 2, 1][:ntier], np.int32)
    tasks, n, core_begin, load = run_lib(lib, ro, row_bytes, unit_rows, tier, alpha, beta, cap, C)
    cost, peer, first, rows = units(ro, row_bytes, unit_rows, tier, alpha, beta)
    assert n == len(cost)
    cap_of_peer = cap[tier] if tier is not None else np.full(R, cap[0], np.int32)
    o_core, o_stripe, o_load = oracle.lpt(cost, peer, cap_of_peer, C)
    assert np.array_equal(load, o_load)                   # same sums in the same order
    # the library lists each core's units in stripe order; map them back by (peer, first_row)
    key = {(int(peer[j]), int(first[j])): j for j in range(n)}
    seen = np.zeros(n, bool)
    for c in range(C):
        prev = -1
        for i in range(core_begin[c], core_begin[c + 1]):
            t = tasks[i]
            j = key[(t.peer, t.first_row)]
            assert not seen[j]
            seen[j] = True
            assert o_core[j] == c and o_stripe[j] == t.stripe and t.rows == rows[j]
            assert t.cost == cost[j]
            assert t.stripe > prev
            prev = t.stripe
    assert seen.all()


def test_lpt_partition_validation(lib):
    ro = np.array([0, 10, 5], np.int32)                  # decreasing
    one = np.ones(1)
    cap = np.ones(1, np.int32)
    core_begin = np.zeros(3, np.int64)
    tasks = (Task * 8)()
    rc = lib.ep_lpt_partition(p(ro), 2, 16, 4, None, p(one), p(one), p(cap), 1, 2,
                              ctypes.cast(tasks, ctypes.c_void_p), 8, p(core_begin), None)
    assert rc == 1 and b"non-decreasing" in lib.ep_last_error()
    ro = np.array([0, 10, 30], np.int32)
    rc = lib.ep_lpt_partition(p(ro), 2, 16, 4, None, p(one), p(one), p(cap), 1, 2,
                              ctypes.cast(tasks, ctypes.c_void_p), 2, p(core_begin), None)
    assert rc == 1 and b"units are needed" in lib.ep_last_error()
    rc = lib.ep_lpt_partition(p(ro), 2, 16, 4, None, p(one), p(np.zeros(1)), p(cap), 1, 2,
                              ctypes.cast(tasks, ctypes.c_void_p), 8, p(core_begin), None)
    assert rc == 1 and b"beta > 0" in lib.ep_last_error()
