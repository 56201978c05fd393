"""GPU parity: every entry point of the C ABI against the CPU oracle, on the five
seeded workloads at their full sizes and on edge cases.

Bars: bit-exact for indices, counts, offsets, positions, dispatched payloads
and combined outputs (the oracle's fp32 chain: the product of pick 0, then a
fused multiply-add per pick in order, then one RNE); route weights within the
bound derived in gpu_util.
Each kernel is fed the oracle's inputs for its stage, so a failure names the
stage.  Calls go through the Python binding straight into the C ABI.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

from gpu_util import (DEV, Case, accuracy_vs_exact, assert_same_bits, bits, check_route_weights,
                      poison_bits, say, to_dev_bits)

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


_CASES = {}


def get_case(name):
    if name not in _CASES:
        _CASES.clear()                      # keep host memory bounded
        _CASES[name] = Case(wl.WORKLOADS[name])
    return _CASES[name]


LAYOUT_KEYS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos",
               "slot_src")


@pytest.mark.parametrize("name", wl.ORDER)
def test_route(epm, name):
    c = get_case(name)
    w = c.w
    say(f"route {w.describe()}")
    idx, wt = epm.ep_route_topk(torch.from_numpy(c.logits).to(DEV), w.k, normalize=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), c.idx)
    check_route_weights(wt.cpu().numpy(), c.wt, c.logits, c.idx, True, w.E)


@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_route_unnormalized(epm, name):
    c = get_case(name)
    w = c.w
    say(f"route normalize=0 {w.describe()}")
    idx, wt = epm.ep_route_topk(torch.from_numpy(c.logits).to(DEV), w.k, normalize=False)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk(c.logits, w.k, 0)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    check_route_weights(wt.cpu().numpy(), o_w, c.logits, o_idx, False, w.E)


@pytest.mark.parametrize("name", wl.ORDER)
def test_layout(epm, name):
    c = get_case(name)
    w = c.w
    say(f"layout {w.describe()}")
    lay = epm.ep_dispatch_layout(torch.from_numpy(c.idx).to(DEV), w.E, w.R)
    assert epm.ep_get_device_error(lay["workspace"]) == epm.EP_OK
    for key in LAYOUT_KEYS:
        np.testing.assert_array_equal(lay[key].cpu().numpy(), c.lay[key], err_msg=key)
    # a second call on the same workspace gives the same answer (state reset)
    lay2 = epm.ep_dispatch_layout(torch.from_numpy(c.idx).to(DEV), w.E, w.R, out=lay)
    np.testing.assert_array_equal(lay2["pos"].cpu().numpy(), c.lay["pos"])


@pytest.mark.parametrize("name", wl.ORDER)
def test_dispatch(epm, name):
    c = get_case(name)
    w = c.w
    say(f"dispatch {w.describe()}")
    send = poison_bits((w.S, w.H))
    epm.ep_dispatch(to_dev_bits(c.x), torch.from_numpy(c.lay["pos"]).to(DEV), send)
    torch.cuda.synchronize()
    got = bits(send)
    del send
    assert np.array_equal(got, c.send), "dispatched payload differs from the oracle"


@pytest.mark.parametrize("name", wl.ORDER)
def test_combine_identity_experts(epm, name):
    """y = the dispatched rows: the oracle's combine, and the round trip to x."""
    c = get_case(name)
    w = c.w
    say(f"combine (identity experts) {w.describe()}")
    out = epm.ep_combine(to_dev_bits(c.send), torch.from_numpy(c.lay["pos"]).to(DEV),
                         torch.from_numpy(c.wt).to(DEV))
    torch.cuda.synchronize()
    got = bits(out)
    assert np.array_equal(got, c.x), "combine(dispatch(x)) != x"
    assert_same_bits(got, oracle.combine(c.send, c.lay["pos"], c.wt), f"combine {name}")


@pytest.mark.parametrize("name", wl.ORDER)
def test_combine_random_experts(epm, name):
    """Distinct random expert outputs and signed weights on every workload
    (the skewed incast one included): the fp32 accumulation, cancellation
    included, bit for bit against the oracle's chain; the distance to the
    exact sum is reported."""
    w = wl.WORKLOADS[name]
    c = get_case(name)
    y = wl.make_rows(w.S, w.H, seed=w.seed + 77)
    wt = (np.random.default_rng(w.seed + 78).random((w.T, w.k), dtype=np.float32)
          - np.float32(0.25))
    say(f"combine (random experts) {w.describe()}")
    out = epm.ep_combine(to_dev_bits(y), torch.from_numpy(c.lay["pos"]).to(DEV),
                         torch.from_numpy(wt).to(DEV))
    torch.cuda.synchronize()
    got = bits(out)
    del out
    assert_same_bits(got, oracle.combine(y, c.lay["pos"], wt), f"combine {name}")
    accuracy_vs_exact(got, oracle.combine_exact(y, c.lay["pos"], wt), f"combine {name}")


def _golden_chain_cases():
    with open(os.path.join(os.path.dirname(__file__), "golden", "combine_chain.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_chain_cases(), ids=lambda c: c["name"])
def test_combine_golden_chain_cases(epm, case):
    """The hand-derived fp32-chain cases (an fma that is not a multiply then an
    add, rounding inside the chain, pick order, signed zeros, fp32 overflow,
    subnormal products) on the GPU: each case's values fill every column of
    every token, at a small shape (one item per wave) and at a large one (the
    batched kernel), and every output must be the hand-derived pattern."""
    k = case["k"]
    for T, H in ((case["T"], 8), (16384 // k * case["T"], 4096)):
        reps = T // case["T"]
        y1 = np.array(case["y"], np.uint16)[:, 0]            # [T0*k]
        pos1 = np.array(case["pos"], np.int32)               # [T0][k]
        w1 = np.array(case["w_bits"], np.uint32).view(np.float32)
        # repetition r uses rows r*T0*k .. : the same values at shifted slots
        n1 = y1.shape[0]
        y = np.repeat(np.tile(y1, reps)[:, None], H, axis=1)
        pos = (np.tile(pos1, (reps, 1)) + (np.arange(reps)[:, None] * n1).repeat(case["T"], 0))
        pos = pos.astype(np.int32)
        wt = np.tile(w1, (reps, 1))
        say(f"combine golden case {case['name']} T={T} H={H} k={k}")
        out = epm.ep_combine(to_dev_bits(y), torch.from_numpy(pos).to(DEV),
                             torch.from_numpy(wt).to(DEV))
        torch.cuda.synchronize()
        want = np.repeat(np.tile(np.array(case["out"], np.uint16), reps)[:, None], H, axis=1)
        assert_same_bits(bits(out), want, f"golden {case['name']} T={T} H={H}")


@pytest.mark.parametrize("name", wl.ORDER)
def test_chain_on_gpu(epm, name):
    """route -> layout -> dispatch -> combine, all on the GPU, one stream."""
    c = get_case(name)
    w = c.w
    say(f"chain {w.describe()}")
    idx, wt = epm.ep_route_topk(torch.from_numpy(c.logits).to(DEV), w.k)
    lay = epm.ep_dispatch_layout(idx, w.E, w.R)
    send = epm.ep_dispatch(to_dev_bits(c.x), lay["pos"])
    out = epm.ep_combine(send, lay["pos"], wt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay["pos"].cpu().numpy(), c.lay["pos"])
    assert np.array_equal(bits(out), c.x)


# ------------------------------------------------------------------ edge cases
EDGE = [
    # T, H, E, R, k, seed
    (1, 8, 1, 1, 1, 1),           # smallest everything
    (3, 16, 4, 2, 2, 2),
    (130, 7176, 64, 8, 6, 3),     # ragged rows (897 vectors) and T % 4 != 0
    (8192, 64, 1024, 8, 4, 4),    # E = 1024: 32 tiles x 1024 experts, bases in the positions launch
    (16384, 16, 1024, 8, 4, 8),   # 65536 counters: separate scan launch, 32 look-back blocks
    (50000, 24, 8, 4, 2, 5),      # 98 tiles, ragged last tile
    (257, 520, 33, 3, 5, 6),      # odd E, odd H/8 = 65
    (64, 4096, 128, 16, 64, 7),   # k = 64 (maximum)
    (3, 1 << 20, 4, 2, 2, 9),     # H = 2^20 (maximum): 2 MiB rows
]


@pytest.mark.parametrize("T,H,E,R,k,seed", EDGE)
def test_edge_shapes(epm, T, H, E, R, k, seed):
    say(f"edge T={T} H={H} E={E} R={R} k={k}")
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = wl.make_rows(T, H, seed)
    o_idx, o_w = oracle.route_topk(logits, k, 1)
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    o_send = oracle.dispatch(x, o_lay["pos"])

    idx, wt = epm.ep_route_topk(torch.from_numpy(logits).to(DEV), k)
    lay = epm.ep_dispatch_layout(torch.from_numpy(o_idx).to(DEV), E, R)
    send = poison_bits((T * k, H))
    epm.ep_dispatch(to_dev_bits(x), torch.from_numpy(o_lay["pos"]).to(DEV), send)
    y = wl.make_rows(T * k, H, seed + 100)
    out_rt = epm.ep_combine(send, torch.from_numpy(o_lay["pos"]).to(DEV),
                            torch.from_numpy(o_w).to(DEV))
    out_y = epm.ep_combine(to_dev_bits(y), torch.from_numpy(o_lay["pos"]).to(DEV),
                           torch.from_numpy(o_w).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    check_route_weights(wt.cpu().numpy(), o_w, logits, o_idx, True, E)
    for key in LAYOUT_KEYS:
        np.testing.assert_array_equal(lay[key].cpu().numpy(), o_lay[key], err_msg=key)
    assert np.array_equal(bits(send), o_send)
    assert np.array_equal(bits(out_rt), x)
    assert_same_bits(bits(out_y), oracle.combine(y, o_lay["pos"], o_w), "combine")


def test_layout_skewed_and_repeated_ids(epm):
    """Every token on the same experts (one hot bucket per pick), and rows that
    repeat an expert: the layout is still the stable counting sort."""
    T, k, E, R = 9000, 4, 16, 4
    idx = np.tile(np.array([3, 3, 15, 0], np.int32), (T, 1))
    idx[::7, 1] = 9
    say("layout skewed/repeated")
    lay = epm.ep_dispatch_layout(torch.from_numpy(idx).to(DEV), E, R)
    o = oracle.dispatch_layout(idx, E, R)
    for key in LAYOUT_KEYS:
        np.testing.assert_array_equal(lay[key].cpu().numpy(), o[key], err_msg=key)


def test_layout_flags_bad_expert_ids(epm):
    T, k, E, R = 300, 2, 8, 2
    rng = np.random.default_rng(9)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[5, 1] = E
    idx[77, 0] = -1
    say("layout with bad ids")
    lay = epm.ep_dispatch_layout(torch.from_numpy(idx).to(DEV), E, R)
    assert epm.ep_get_device_error(lay["workspace"]) == epm.EP_ERR_DEVICE
    pos = lay["pos"].cpu().numpy()
    assert pos[5, 1] == -1 and pos[77, 0] == -1
    ok = (idx >= 0) & (idx < E)
    flat_ok = idx[ok]
    # the valid picks form the stable counting sort of the valid ids
    perm = np.argsort(flat_ok, kind="stable")
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    np.testing.assert_array_equal(pos[ok], inv)
    # and the next good call clears the error
    lay = epm.ep_dispatch_layout(torch.from_numpy(np.where(ok, idx, 0).astype(np.int32)).to(DEV),
                                 E, R, out=lay)
    assert epm.ep_get_device_error(lay["workspace"]) == epm.EP_OK


def test_streams_are_respected(epm):
    """Work enqueued on a side stream is ordered on that stream."""
    c = get_case("decode")
    w = c.w
    say("side stream chain")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        logits = torch.from_numpy(c.logits).to(DEV)
        x = to_dev_bits(c.x)
        idx, wt = epm.ep_route_topk(logits, w.k, stream=s)
        lay = epm.ep_dispatch_layout(idx, w.E, w.R, stream=s)
        send = epm.ep_dispatch(x, lay["pos"], stream=s)
        out = epm.ep_combine(send, lay["pos"], wt, stream=s)
    s.synchronize()
    assert np.array_equal(bits(out), c.x)


def test_concurrent_host_threads_on_separate_streams(epm):
    """Calls on different streams with separate buffers and workspaces are
    independent: two host threads run the whole chain at once, each on its
    own stream (ctypes releases the interpreter lock during the calls), and
    each gets the oracle's answer."""
    import threading
    c = get_case("glm45air")
    w = c.w
    results, errors = {}, []
    logits = torch.from_numpy(c.logits).to(DEV)
    x = to_dev_bits(c.x)
    torch.cuda.synchronize()

    def worker(i):
        try:
            s = torch.cuda.Stream()
            for _ in range(5):
                idx, wt = epm.ep_route_topk(logits, w.k, stream=s)
                lay = epm.ep_dispatch_layout(idx, w.E, w.R, stream=s)
                send = epm.ep_dispatch(x, lay["pos"], stream=s)
                out = epm.ep_combine(send, lay["pos"], wt, stream=s)
            s.synchronize()
            results[i] = (bits(out), lay["pos"].cpu().numpy())
        except Exception as e:            # reported below, in the test's thread
            errors.append(repr(e))

    say("two host threads, two streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i in range(2):
        out, pos = results[i]
        assert np.array_equal(out, c.x)
        np.testing.assert_array_equal(pos, c.lay["pos"])


# Gathers reading over 64 MiB with rows of whole 1 KiB segments take the
# batched combine (outputs held back in registers and stored a batch at a
# time on one workgroup per CU): full and partial batches, runtime k.
BATCHED = [
    # T, H, E, R, k, seed
    (5000, 1536, 64, 8, 8, 41),      # a single partial batch
    (4096, 4096, 64, 16, 6, 42),     # k = 6 (compile-time): one full batch and a partial one
    (20000, 1024, 256, 32, 8, 43),   # one full batch and a partial one
    (8192, 2048, 64, 8, 4, 44),      # k = 4 (compile-time)
    (9000, 4096, 32, 8, 2, 45),      # k = 2 (compile-time)
    (5000, 2048, 64, 8, 5, 46),      # runtime-k path (picks loaded in groups of 4)
]


@pytest.mark.parametrize("T,H,E,R,k,seed", BATCHED)
def test_combine_batched_sizes(epm, T, H, E, R, k, seed):
    rng = np.random.default_rng(seed)
    o_idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    pos = oracle.dispatch_layout(o_idx, E, R)["pos"]
    y = wl.make_rows(T * k, H, seed + 1)
    wt = rng.random((T, k), dtype=np.float32) - np.float32(0.25)
    say(f"combine (batched sizes) T={T} H={H} k={k}")
    d_y, d_pos = to_dev_bits(y), torch.from_numpy(pos).to(DEV)
    out = epm.ep_combine(d_y, d_pos, torch.from_numpy(wt).to(DEV))
    gx = epm.ep_dispatch_grad(d_y, d_pos)
    torch.cuda.synchronize()
    assert_same_bits(bits(out), oracle.combine(y, pos, wt), "combine")
    assert_same_bits(bits(gx), oracle.dispatch_grad(y, pos), "dispatch_grad")


def test_combine_batched_skips_picks_outside(epm):
    """pos entries outside [0, T*k) contribute nothing, also in the batched
    combine: in a batch that is otherwise full and in the partial one."""
    T, H, E, R, k = 4096, 4096, 128, 16, 8
    rng = np.random.default_rng(44)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    pos = oracle.dispatch_layout(o_idx, E, R)["pos"]
    y = wl.make_rows(T * k, H, 45)
    bad = pos.copy()
    picks = [(5, 2, -1), (1000, 0, T * k), (4000, 7, T * k + 9)]
    lost = [pos[t, j] for t, j, _ in picks]
    for t, j, v in picks:
        bad[t, j] = v
    say("combine (batched sizes) with picks outside the buffer")
    out = epm.ep_combine(to_dev_bits(y), torch.from_numpy(bad).to(DEV),
                         torch.from_numpy(o_w).to(DEV))
    torch.cuda.synchronize()
    y0 = y.copy()
    y0[lost] = 0
    assert_same_bits(bits(out), oracle.combine(y0, pos, o_w), "combine with picks outside")


def test_dispatch_large_skips_picks_outside(epm):
    """A pos entry outside [0, T*k) writes nothing, also at sizes that take the
    capped grid (whole 1 KiB segments, and a ragged row of 513 vectors)."""
    for T, H, E, R, k, seed in ((4096, 4096, 128, 16, 8, 46), (4096, 4104, 64, 8, 6, 47)):
        rng = np.random.default_rng(seed)
        o_idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
        pos = oracle.dispatch_layout(o_idx, E, R)["pos"]
        x = wl.make_rows(T, H, seed + 1)
        bad = pos.copy()
        lost = [pos[3, 1], pos[2000, 0], pos[T - 1, k - 1]]
        bad[3, 1], bad[2000, 0], bad[T - 1, k - 1] = -1, T * k, T * k + 77
        say(f"dispatch (large) T={T} H={H} k={k}, picks outside the buffer")
        send = poison_bits((T * k, H))
        epm.ep_dispatch(to_dev_bits(x), torch.from_numpy(bad).to(DEV), send)
        torch.cuda.synchronize()
        ref = oracle.dispatch(x, pos)
        ref[lost] = 0xFFFF
        assert np.array_equal(bits(send), ref)


def test_route_unaligned_logits_take_the_scalar_path(epm):
    """Logits 4- but not 16-byte aligned (and E % 4 != 0) read one float per
    load; the picks and weights are the same as the oracle's."""
    for T, E, k, norm in ((1000, 256, 8, 1), (333, 64, 6, 0), (77, 33, 5, 1)):
        rng = np.random.default_rng(T + E)
        logits = rng.standard_normal((T, E), dtype=np.float32)
        flat = torch.empty(T * E + 1, dtype=torch.float32, device=DEV)
        d = flat[1:].view(T, E)                    # 4 bytes past a 256-byte boundary
        d.copy_(torch.from_numpy(logits))
        say(f"route with unaligned logits T={T} E={E} k={k} normalize={norm}")
        idx, w = epm.ep_route_topk(d, k, bool(norm))
        torch.cuda.synchronize()
        o_idx, o_w = oracle.route_topk(logits, k, norm)
        np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
        check_route_weights(w.cpu().numpy(), o_w, logits, o_idx, bool(norm), E)


def test_route_ties_pick_the_lowest_expert(epm):
    """Logits drawn from five values (-0.0 and +0.0 among them) tie in every
    row; row 0 holds one value throughout and row 1 alternates -0.0 and
    +0.0.  Equal logits go to the lowest expert id and -0.0 ranks equal to
    +0.0, so every pick is unique and equals the oracle's, on the vector and
    scalar load paths and at group sizes G = 8, 16, 32 and 64."""
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
    for T, E, k, norm in ((1000, 256, 8, 1), (500, 128, 8, 0), (300, 64, 6, 1), (200, 33, 5, 1),
                          (100, 512, 8, 1), (100, 1024, 4, 0)):
        rng = np.random.default_rng(T * E + k)
        logits = vals[rng.integers(0, len(vals), (T, E))]
        logits[0, :] = np.float32(0.25)
        logits[1, :] = np.float32(-0.0)
        logits[1, ::2] = np.float32(0.0)
        say(f"route with ties T={T} E={E} k={k} normalize={norm}")
        idx, w = epm.ep_route_topk(torch.from_numpy(logits).to(DEV), k, bool(norm))
        torch.cuda.synchronize()
        o_idx, o_w = oracle.route_topk(logits, k, norm)
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(got, o_idx)
        np.testing.assert_array_equal(got[0], np.arange(k))
        np.testing.assert_array_equal(got[1], np.arange(k))
        check_route_weights(w.cpu().numpy(), o_w, logits, o_idx, bool(norm), E)


def test_maximum_slot_count(epm):
    """T*k just under the 2^30 limit (T = 134,000,000 tokens, k = 8, E = 16,
    H = 8): the layout's separate look-back scan over ~4,000 blocks, and every
    output checked by properties on the GPU, plus sampled tokens against the
    oracle.  About 50 GB of device memory."""
    T, E, R, k, H = 134_000_000, 16, 4, 8, 8
    S = T * k
    assert S < (1 << 30)
    g = torch.Generator(device=DEV)
    g.manual_seed(1_000_003)
    say(f"maximum slot count T={T} k={k} E={E}: route")
    logits = torch.randn((T, E), generator=g, dtype=torch.float32, device=DEV)
    idx, w = epm.ep_route_topk(logits, k)
    torch.cuda.synchronize()
    sample = torch.randint(0, T, (10_000,), generator=g, device=DEV)
    o_idx, o_w = oracle.route_topk(logits[sample].cpu().numpy(), k, 1)
    np.testing.assert_array_equal(idx[sample].cpu().numpy(), o_idx)
    check_route_weights(w[sample].cpu().numpy(), o_w, logits[sample].cpu().numpy(), o_idx, True, E)
    del logits

    say("maximum slot count: layout")
    lay = epm.ep_dispatch_layout(idx, E, R)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(lay["workspace"]) == epm.EP_OK
    flat = idx.reshape(-1)
    counts = torch.bincount(flat, minlength=E)
    assert torch.equal(lay["expert_counts"].long(), counts)
    offs = torch.zeros(E + 1, dtype=torch.int64, device=DEV)
    offs[1:] = torch.cumsum(counts, 0)
    assert torch.equal(lay["expert_offsets"].long(), offs)
    pos = lay["pos"].reshape(-1).long()
    src = lay["slot_src"].long()
    # pos and slot_src are inverse permutations of [0, S)
    assert torch.equal(src[pos], torch.arange(S, device=DEV))
    del pos
    # slots in expert-major order, ascending source slot inside each expert
    e_of = flat[src]
    assert bool((e_of[1:] >= e_of[:-1]).all())
    same = e_of[1:] == e_of[:-1]
    assert bool((src[1:][same] > src[:-1][same]).all())
    del e_of, same, src, flat
    torch.cuda.empty_cache()

    say("maximum slot count: dispatch and combine")
    # finite rows (N(0, 1) in bf16), like the workloads': the round trip is exact for them
    x = torch.randn((T, H), generator=g, dtype=torch.bfloat16, device=DEV)
    send = epm.ep_dispatch(x, lay["pos"])
    out = epm.ep_combine(send, lay["pos"], w)
    torch.cuda.synchronize()
    xs = x.view(torch.int16)
    assert torch.equal(out.view(torch.int16), xs), "combine(dispatch(x)) != x"
    rows = lay["pos"][sample].long()                       # [n][k] slots of sampled tokens
    got = send.view(torch.int16)[rows.reshape(-1)].reshape(len(sample), k, H)
    assert torch.equal(got, xs[sample][:, None, :].expand(-1, k, -1))
