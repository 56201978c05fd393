"""GPU parity of rank-level token coalescing (ep_rank_coalesce) against the
CPU oracle, bit for bit, and of the coalesced dispatch it feeds.

RailWave sec. 3.1-3.2: the transfer records of a destination keep the
backend's token coalescing, and one record may carry several destinations of
a token -- read as one send record per (token, destination rank).  The
receiver's expansion of the records into the expert layout (pick (t, j)'s
row = record row_of_pick[t][j]) must give the uncoalesced dispatch."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

from gpu_util import DEV, bits, poison_bits, say, to_dev_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


def check(epm, idx, E, R, x=None):
    T, k = idx.shape
    got = epm.ep_rank_coalesce(torch.from_numpy(idx).to(DEV), E, R)
    got["row_src"][:] = -7
    got = epm.ep_rank_coalesce(torch.from_numpy(idx).to(DEV), E, R, out=got)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(got["workspace"]) == epm.EP_OK
    ref = oracle.rank_coalesce(idx, E, R)
    C = int(ref["rank_offsets"][R])
    for key in ("rank_counts", "rank_offsets", "row_of_pick", "send_pos"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    row_src = got["row_src"].cpu().numpy()
    np.testing.assert_array_equal(row_src[:C], ref["row_src"])
    assert np.all(row_src[C:] == -7)
    np.testing.assert_array_equal(got["row_experts"].cpu().numpy()[:C].view(np.uint64),
                                  ref["row_experts"])
    if x is not None:
        H = x.shape[1]
        send = poison_bits((T * k, H))
        epm.ep_dispatch(to_dev_bits(x), got["send_pos"], send)
        torch.cuda.synchronize()
        sb = bits(send)
        assert np.array_equal(sb[:C], x[ref["row_src"]]), "coalesced dispatch"
        assert np.all(sb[C:] == 0xFFFF), "rows beyond the records were written"
        # the receiver's expansion into the expert layout equals the plain dispatch
        lay = oracle.dispatch_layout(idx, E, R)
        expanded = np.empty((T * k, H), np.uint16)
        expanded[lay["pos"].reshape(-1)] = sb[ref["row_of_pick"].reshape(-1)]
        assert np.array_equal(expanded, oracle.dispatch(x, lay["pos"]))
    return C


@pytest.mark.parametrize("name", wl.ORDER)
def test_coalesce_workloads(epm, name):
    w = wl.WORKLOADS[name]
    idx, _ = oracle.route_topk(wl.make_logits(w), w.k, 1)
    say(f"rank coalesce {w.describe()}")
    x = wl.make_rows(w.T, w.H, w.seed) if w.T * w.H <= 4096 * 7168 else None
    C = check(epm, idx, w.E, w.R, x)
    print(f"[gpu-test] {name}: {C} records for {w.T * w.k} picks ({C / (w.T * w.k):.3f})")


COALESCE_EDGE = [
    # T, E, R, k, seed
    (1, 1, 1, 1, 1301),
    (3, 8, 2, 4, 1302),          # every pick of a token on few ranks
    (700, 64, 8, 6, 1303),       # runtime k, five tiles
    (5000, 1024, 16, 8, 1304),   # 64 local experts per rank, E = 1024
    (2000, 1000, 1000, 8, 1305), # one expert per rank, R = 1000
    (64, 64, 1, 64, 1306),       # k = 64 on one rank: one record per token
]


@pytest.mark.parametrize("T,E,R,k,seed", COALESCE_EDGE)
def test_coalesce_edge_shapes(epm, T, E, R, k, seed):
    rng = np.random.default_rng(seed)
    idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    say(f"rank coalesce edge T={T} E={E} R={R} k={k}")
    check(epm, idx, E, R, wl.make_rows(T, 64, seed))


def test_coalesce_reports_bad_ids(epm):
    T, E, R, k = 512, 64, 8, 4
    rng = np.random.default_rng(1310)
    idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    idx[7, 2], idx[300, 0] = E + 3, -1
    say("rank coalesce with ids outside [0, E)")
    got = epm.ep_rank_coalesce(torch.from_numpy(idx).to(DEV), E, R)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(got["workspace"]) == epm.EP_ERR_DEVICE
    rop = got["row_of_pick"].cpu().numpy()
    assert rop[7, 2] == -1 and rop[300, 0] == -1
    # a good call on the same workspace reports OK again
    good = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32)
    epm.ep_rank_coalesce(torch.from_numpy(good).to(DEV), E, R, out=got)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(got["workspace"]) == epm.EP_OK


@pytest.mark.parametrize("name", ["decode", "glm45air", "dsv3"])
def test_coalesced_exchange_end_to_end(epm, name):
    """Sender and receiver of the coalesced exchange on one GPU: the records
    (ep_rank_coalesce + ep_dispatch(send_pos)) of every rank, expanded by
    ep_expand_records into that rank's local experts' slots, equal the rank's
    segment of the plain dispatch, and its slot positions equal the oracle's."""
    w = wl.WORKLOADS[name]
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    L = E // R
    idx, _ = oracle.route_topk(wl.make_logits(w), k, 1)
    x = wl.make_rows(T, H, w.seed)
    d_idx, d_x = torch.from_numpy(idx).to(DEV), to_dev_bits(x)
    say(f"coalesced exchange end to end {w.describe()}")
    co = epm.ep_rank_coalesce(d_idx, E, R)
    records = epm.ep_dispatch(d_x, co["send_pos"])
    lay = epm.ep_dispatch_layout(d_idx, E, R)
    plain = epm.ep_dispatch(d_x, lay["pos"])
    torch.cuda.synchronize()
    ro = co["rank_offsets"].cpu().numpy()
    pro = lay["rank_offsets"].cpu().numpy()
    masks = co["row_experts"]
    ref = oracle.rank_coalesce(idx, E, R)
    for r in range(R):
        a, b = int(ro[r]), int(ro[r + 1])
        if a == b:
            continue
        n = int(pro[r + 1] - pro[r])
        got = epm.ep_expand_records(records[a:b], masks[a:b], L, n)
        torch.cuda.synchronize()
        assert epm.ep_get_device_error(got["workspace"]) == epm.EP_OK, f"rank {r}"
        assert torch.equal(got["recv"].view(torch.int16), plain[pro[r]:pro[r + 1]].view(torch.int16)), f"rank {r}"
        e_ref = oracle.expand_records(ref["row_experts"][a:b], L)
        np.testing.assert_array_equal(got["pos"].cpu().numpy(), e_ref["pos"], err_msg=f"rank {r}")
        np.testing.assert_array_equal(got["expert_counts"].cpu().numpy(),
                                      lay["expert_counts"][r * L:(r + 1) * L].cpu().numpy())
    # the plain dispatch itself against the oracle
    assert np.array_equal(bits(plain), oracle.dispatch(x, oracle.dispatch_layout(idx, E, R)["pos"]))


def test_expand_records_reports_overflow(epm):
    rows = to_dev_bits(wl.make_rows(6, 64, 1420))
    masks = torch.tensor([3, 1, 2, 4, 1, 6], dtype=torch.int64, device=DEV)    # 9 slots, L = 3
    say("expand records into a buffer that is too small")
    got = epm.ep_expand_records(rows, masks, 3, 7)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(got["workspace"]) == epm.EP_ERR_DEVICE
    got = epm.ep_expand_records(rows, masks, 3, 9, out=None)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(got["workspace"]) == epm.EP_OK
