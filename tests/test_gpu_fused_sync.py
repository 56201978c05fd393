"""GPU parity of the fused mode's Data-as-Flag variants
(ep_fused_dispatch_combine_sync; UBEP sec. 3.4, Fig. 6): row flags, a
per-batch checksum and sentinel polling, against the CPU oracle and the
default mode, on every workload, edge shapes, alternating modes on one
workspace, the sentinel collision and the bounded-wait path."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

from gpu_util import DEV, Case, assert_same_bits, bits, say, to_dev_bits

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos")
MODES = {1: "row flags", 2: "checksum", 3: "sentinel", 4: "chunk flags"}
SENTINEL_WORD_HALF = 0x7FA5          # bf16; the reserved 32-bit word is two of them


@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


def check(fz, x_bits, idx, wt, E, R, H, sync, epoch=None):
    o_lay = oracle.dispatch_layout(idx, E, R)
    for key in LAYOUT_KEYS:
        np.testing.assert_array_equal(fz[key].cpu().numpy(), o_lay[key], err_msg=key)
    rows = fz["send_rows"].cpu().numpy()
    o_send = oracle.dispatch(x_bits, o_lay["pos"])
    assert np.array_equal(rows[:, :2 * H].copy().view(np.uint16), o_send), "payload"
    if sync == 1 and epoch is not None:
        assert np.array_equal(rows[:, 2 * H:2 * H + 16],
                              oracle.fused_trailers(epoch, o_lay["slot_src"])), "trailers"
    if sync == 4 and epoch is not None:
        nchunk = -(-2 * H // 1024)
        flags = rows[:, 2 * H + 16:2 * H + 16 + 8 * nchunk].copy().view(np.uint64)
        assert np.all(flags == np.uint64(epoch)), "chunk flags"
    # a NaN input gives NaN outputs whose bit patterns the format leaves open
    assert_same_bits(bits(fz["out"]), oracle.combine(o_send, o_lay["pos"], wt), "out")


@pytest.mark.parametrize("sync", sorted(MODES))
@pytest.mark.parametrize("name", wl.ORDER)
def test_sync_modes_match_oracle(epm, name, sync):
    w = wl.WORKLOADS[name]
    c = Case(w)
    say(f"fused sync={MODES[sync]} {w.describe()}")
    x = to_dev_bits(c.x)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    fz = epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, want_epoch=True, sync=sync)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    check(fz, c.x, c.idx, c.wt, w.E, w.R, w.H, sync, fz["epoch"])
    assert np.array_equal(bits(fz["out"]), c.x)     # identity experts: the round trip


SYNC_EDGE = [
    (1, 8, 1, 1, 1, 31),
    (5, 16, 4, 2, 2, 32),
    (130, 7176, 64, 8, 6, 33),     # ragged rows, runtime-k path
    (3000, 520, 33, 3, 5, 34),
    (64, 4096, 128, 16, 64, 35),   # k = 64
    (20000, 256, 16, 4, 8, 36),    # many items, small rows
    (3, 1 << 20, 4, 2, 2, 37),     # H = 2^20 (maximum): 2 MiB rows
]


@pytest.mark.parametrize("sync", sorted(MODES))
@pytest.mark.parametrize("T,H,E,R,k,seed", SYNC_EDGE)
def test_sync_modes_edge_shapes(epm, T, H, E, R, k, seed, sync):
    rng = np.random.default_rng(seed)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    x = wl.make_rows(T, H, seed)
    say(f"fused sync={MODES[sync]} edge T={T} H={H} E={E} R={R} k={k}")
    fz = epm.ep_fused_dispatch_combine(to_dev_bits(x), torch.from_numpy(o_idx).to(DEV),
                                       torch.from_numpy(o_w).to(DEV), E, R, want_epoch=True,
                                       sync=sync)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    check(fz, x, o_idx, o_w, E, R, H, sync, fz["epoch"])


def test_modes_alternate_on_one_workspace(epm):
    """Every mode after every other on one workspace and one set of rows, on
    new inputs each call: stale trailers, checksum words and sentinels of
    other calls are never taken for this call's."""
    w = wl.WORKLOADS["glm45air"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    for i, sync in enumerate([0, 1, 2, 3, 4, 0, 4, 3, 2, 1, 3, 4, 4, 2, 2]):
        x_bits = wl.make_rows(w.T, w.H, seed=700 + i)
        say(f"alternating call {i} sync={sync}")
        epm.ep_fused_dispatch_combine(to_dev_bits(x_bits), idx, wt, w.E, w.R, out=fz, sync=sync)
        torch.cuda.synchronize()
        assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
        assert np.array_equal(bits(fz["out"]), x_bits), f"call {i} sync={sync}"


@pytest.mark.parametrize("sync", [2, 3, 4])
def test_sync_modes_back_to_back_without_host_sync(epm, sync):
    w = wl.WORKLOADS["dsv3"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    x = to_dev_bits(c.x)
    say(f"fused sync={MODES[sync]} back-to-back x20")
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    for _ in range(20):
        epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz, sync=sync)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    assert np.array_equal(bits(fz["out"]), c.x)


@pytest.mark.parametrize("name,calls", [("dsv3", 200), ("incast", 60), ("decode", 400),
                                        ("glm45air", 200)])
def test_every_mode_long_back_to_back(epm, name, calls):
    """Long runs without host synchronisation, every readiness mode in turn on
    one workspace (epochs keep growing across modes): every 20th call the
    device error word is clear and the output is the round trip, then the
    output is zeroed so the next check sees only later calls' work.  The
    decode-like batch splits its rows into parts in item-event mode (and not
    in the others), the GLM-like one splits each 8 KiB row into two 4-chunk
    runs; both keep their rows cached."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    x = to_dev_bits(inp["x"])
    idx, wt = epm.ep_route_topk(torch.from_numpy(inp["logits"]).to(DEV), w.k)
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    for sync in (0, *MODES):
        say(f"fused sync={MODES.get(sync, 'item events')} {name} x{calls}")
        for c in range(calls):
            epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz, sync=sync)
            if (c + 1) % 20 == 0:
                torch.cuda.synchronize()
                assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK, (sync, c)
                assert torch.equal(fz["out"].view(torch.int16), x.view(torch.int16)), (sync, c)
                fz["out"].zero_()


def test_sentinel_collision_is_reported(epm):
    """UBEP sec. 3.4: data equal to the sentinel cannot be told from no data.
    A token whose leading 16 bytes hold the reserved 32-bit word makes the
    sentinel mode report EP_ERR_DEVICE (its waits end early, never hang);
    the next call on the workspace is correct, and the other modes take the
    same data."""
    T, H, E, R, k = 512, 256, 16, 4, 4
    rng = np.random.default_rng(41)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    x = wl.make_rows(T, H, 42)
    bad = x.copy()
    bad[77, 4:6] = SENTINEL_WORD_HALF
    idx = torch.from_numpy(o_idx).to(DEV)
    wt = torch.from_numpy(o_w).to(DEV)
    fz = epm.fused_outputs(T, H, k, E, R, DEV)
    say("sentinel collision")
    epm.ep_fused_dispatch_combine(to_dev_bits(bad), idx, wt, E, R, out=fz, sync=3)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_ERR_DEVICE
    say("sentinel after a collision")
    epm.ep_fused_dispatch_combine(to_dev_bits(x), idx, wt, E, R, out=fz, sync=3)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    check(fz, x, o_idx, o_w, E, R, H, 3)
    # the reserved word is two bf16 signalling NaNs: combine passes NaNs on
    for sync in (0, 1, 2, 4):
        say(f"reserved word through sync={sync}")
        epm.ep_fused_dispatch_combine(to_dev_bits(bad), idx, wt, E, R, out=fz, sync=sync,
                                      want_epoch=True)
        torch.cuda.synchronize()
        assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
        check(fz, bad, o_idx, o_w, E, R, H, sync, fz["epoch"])


@pytest.mark.parametrize("sync", sorted(MODES))
def test_sync_modes_bounded_waits_recover(epm, sync):
    w = wl.WORKLOADS["dsv3"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    x = to_dev_bits(c.x)
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    say(f"fused sync={MODES[sync]} spin_limit=1")
    epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz, spin_limit=1, sync=sync)
    rc = epm.ep_get_device_error(fz["workspace"])
    assert rc in (epm.EP_OK, epm.EP_ERR_TIMEOUT)
    say(f"fused sync={MODES[sync]} after a bounded-wait call")
    epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz, sync=sync)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    assert np.array_equal(bits(fz["out"]), c.x)


def test_invalid_sync_is_rejected(epm):
    T, H, E, R, k = 8, 16, 4, 2, 2
    fz = epm.fused_outputs(T, H, k, E, R, DEV)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    wt = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    for bad in (-1, 5):
        with pytest.raises(epm.EpError):
            epm.ep_fused_dispatch_combine(x, idx, wt, E, R, out=fz, sync=bad)
