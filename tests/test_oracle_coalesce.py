"""Pins of the oracle's rank-level token coalescing and exchange waves.

RailWave sec. 3.1-3.2: the transfer records of a destination keep the
backend's token coalescing, and one record may carry several destinations of
the same token.  Read as one send record per (token, destination rank), with
the bit mask of the rank's local experts the token picked; records are
rank-major, then in ascending token order.  RailWave sec. 3.2, eq. (10): wave
k = 1..N-1 of the cyclic pairwise exchange sends from node s to (s + k) mod N;
App. A.6, Table 8 lists four 4-node schedules and their peak incast degrees.

Pins: a hand-derived example; brute force over Python sets on random
routings; the special cases E == R (each rank one expert: the records are the
expert layout's slots, pinned separately) and R == 1 (one record per token);
the page's Table 8 (the permutation schedule and all four incast rows); every
ordered pair exactly once per round.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_coalesce_hand_example():
    g = load("coalesce_small.json")
    c = oracle.rank_coalesce(np.array(g["topk_idx"], np.int32), g["E"], g["R"])
    for key in ("rank_counts", "rank_offsets", "row_of_pick", "send_pos", "row_src"):
        np.testing.assert_array_equal(c[key], np.array(g[key]), err_msg=key)
    np.testing.assert_array_equal(c["row_experts"], np.array(g["row_experts"], np.uint64))


def random_idx(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("seed", range(10))
def test_coalesce_against_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8]))
    L = int(rng.integers(1, 9))
    E, T = R * L, int(rng.integers(1, 60))
    k = int(rng.integers(1, E + 1))
    idx = random_idx(rng, T, E, k)
    c = oracle.rank_coalesce(idx, E, R)
    # the records: the set of (token, rank) pairs, rank-major then token order
    rec = sorted({(int(e) // L, t) for t in range(T) for e in idx[t]})
    C = len(rec)
    assert c["rank_offsets"][R] == C
    np.testing.assert_array_equal(c["rank_counts"], [sum(1 for r, _ in rec if r == q) for q in range(R)])
    np.testing.assert_array_equal(c["rank_offsets"], np.concatenate([[0], np.cumsum(c["rank_counts"])]))
    np.testing.assert_array_equal(c["row_src"], [t for _, t in rec])
    row = {rt: i for i, rt in enumerate(rec)}
    for t in range(T):
        seen = set()
        for j in range(k):
            r = int(idx[t, j]) // L
            assert c["row_of_pick"][t, j] == row[(r, t)]
            assert c["send_pos"][t, j] == (row[(r, t)] if r not in seen else -1)
            seen.add(r)
    for i, (r, t) in enumerate(rec):
        mask = 0
        for e in idx[t]:
            if int(e) // L == r:
                mask |= 1 << (int(e) % L)
        assert int(c["row_experts"][i]) == mask
    # every record is written exactly once by the first-pick positions
    sp = c["send_pos"][c["send_pos"] >= 0]
    np.testing.assert_array_equal(np.sort(sp), np.arange(C))
    # each pick's local expert is in exactly one record's mask: popcounts sum to T*k
    assert sum(bin(int(m)).count("1") for m in c["row_experts"]) == T * k


@pytest.mark.parametrize("seed", range(4))
def test_coalesce_one_expert_per_rank_is_the_expert_layout(seed):
    rng = np.random.default_rng(600 + seed)
    T, E, k = 50, 12, 4
    idx = random_idx(rng, T, E, k)
    c = oracle.rank_coalesce(idx, E, E)
    lay = oracle.dispatch_layout(idx, E, E)
    np.testing.assert_array_equal(c["rank_counts"], lay["expert_counts"])
    np.testing.assert_array_equal(c["rank_offsets"], lay["expert_offsets"])
    np.testing.assert_array_equal(c["row_of_pick"], lay["pos"])
    np.testing.assert_array_equal(c["send_pos"], lay["pos"])
    np.testing.assert_array_equal(c["row_src"], lay["slot_src"] // k)
    assert np.all(c["row_experts"] == 1)


def test_coalesce_single_rank_is_one_record_per_token():
    rng = np.random.default_rng(7)
    T, E, k = 33, 40, 5
    idx = random_idx(rng, T, E, k)
    c = oracle.rank_coalesce(idx, E, 1)
    assert c["rank_offsets"][1] == T
    np.testing.assert_array_equal(c["row_of_pick"], np.repeat(np.arange(T)[:, None], k, 1))
    np.testing.assert_array_equal(c["send_pos"][:, 0], np.arange(T))
    assert np.all(c["send_pos"][:, 1:] == -1)
    for t in range(T):
        assert int(c["row_experts"][t]) == sum(1 << int(e) for e in idx[t])


def test_coalesced_dispatch_expands_to_the_expert_layout():
    """The receiver's view: every pick's expert row equals the token's record
    row, so expanding the coalesced send buffer by (row_of_pick -> pos) gives
    the uncoalesced dispatch bit for bit."""
    rng = np.random.default_rng(8)
    T, E, R, k, H = 40, 32, 4, 6, 16
    idx = random_idx(rng, T, E, k)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    c = oracle.rank_coalesce(idx, E, R)
    send_c = x[c["row_src"]]                     # each record holds its token's row
    lay = oracle.dispatch_layout(idx, E, R)
    expanded = np.empty((T * k, H), np.uint16)
    expanded[lay["pos"].reshape(-1)] = send_c[c["row_of_pick"].reshape(-1)]
    np.testing.assert_array_equal(expanded, oracle.dispatch(x, lay["pos"]))


def test_coalesce_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.rank_coalesce(np.array([[0, 16]], np.int32), 16, 2)     # id outside [0, E)
    with pytest.raises(ValueError):
        oracle.rank_coalesce(np.array([[0]], np.int32), 130, 1)        # 130 local experts > 64
    with pytest.raises(ValueError):
        oracle.rank_coalesce(np.array([[0]], np.int32), 10, 3)         # E % R != 0


def test_exchange_waves_match_table8():
    g = load("railwave_table8.json")
    N = g["nodes"]
    np.testing.assert_array_equal(oracle.exchange_waves(N), g["schedules"]["Permutation"]["waves"])
    for name, sch in g["schedules"].items():
        got = [oracle.incast_degree(w) for w in sch["waves"]]
        assert got == sch["peak_incast"], name


@pytest.mark.parametrize("N", [1, 2, 3, 4, 7, 8, 16])
def test_exchange_waves_cover_every_pair_once(N):
    peer = oracle.exchange_waves(N)
    assert peer.shape == (N - 1, N)
    pairs = [(s, int(peer[w, s])) for w in range(N - 1) for s in range(N)]
    assert sorted(pairs) == sorted((s, d) for s in range(N) for d in range(N) if d != s)
    for w in range(N - 1):
        assert sorted(peer[w]) == list(range(N))        # one sender per receiver
        assert oracle.incast_degree(peer[w]) == 1


def test_expand_records_hand_example():
    # masks 0b011, 0b100, 0b001 over L = 3 local experts:
    # expert 0 <- records 0, 2; expert 1 <- record 0; expert 2 <- record 1
    e = oracle.expand_records(np.array([3, 4, 1], np.uint64), 3)
    np.testing.assert_array_equal(e["expert_counts"], [2, 1, 1])
    np.testing.assert_array_equal(e["expert_offsets"], [0, 2, 3, 4])
    np.testing.assert_array_equal(e["pos"], [[0, 2, -1], [-1, -1, 3], [1, -1, -1]])


@pytest.mark.parametrize("seed", range(6))
def test_expanding_each_ranks_records_gives_its_expert_segment(seed):
    """The receiver's side: rank r's records (its segment of the coalesced
    send buffer, with their masks) expanded into its local experts' slots give
    exactly rank r's segment of the plain dispatch, and its expert counts."""
    rng = np.random.default_rng(700 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    L = int(rng.choice([1, 3, 8, 16]))
    E, T, H = R * L, int(rng.integers(1, 80)), 8
    k = int(rng.integers(1, E + 1))
    idx = random_idx(rng, T, E, k)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    c = oracle.rank_coalesce(idx, E, R)
    records = x[c["row_src"]]
    lay = oracle.dispatch_layout(idx, E, R)
    send = oracle.dispatch(x, lay["pos"])
    for r in range(R):
        a, b = c["rank_offsets"][r], c["rank_offsets"][r + 1]
        e = oracle.expand_records(c["row_experts"][a:b], L)
        np.testing.assert_array_equal(e["expert_counts"], lay["expert_counts"][r * L:(r + 1) * L])
        n = int(e["expert_offsets"][L])
        recv = np.empty((n, H), np.uint16)
        for rec in range(b - a):
            for i in range(L):
                if e["pos"][rec, i] >= 0:
                    recv[e["pos"][rec, i]] = records[a + rec]
        lo, hi = lay["rank_offsets"][r], lay["rank_offsets"][r + 1]
        np.testing.assert_array_equal(recv, send[lo:hi])


def test_expand_records_rejects_a_bit_past_the_last_expert():
    with pytest.raises(ValueError):
        oracle.expand_records(np.array([1 << 5], np.uint64), 4)
