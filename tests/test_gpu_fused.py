"""GPU parity of the fused flag-in-payload mode (ep_fused_dispatch_combine):
layout outputs, payload rows, trailers and the combined output against the
CPU oracle, equality with the three-launch path, epochs across calls, the
bounded-wait error path and bad expert ids."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

from gpu_util import DEV, Case, assert_same_bits, bits, say, to_dev_bits

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos")


@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


def split_rows(rows: np.ndarray, H: int):
    payload = rows[:, :2 * H].copy().view(np.uint16)
    trailer = rows[:, 2 * H:2 * H + 16]
    return payload, trailer


def check_fused(epm, fz, x_bits, idx, wt, E, R, H, k, expect_out=None):
    o_lay = oracle.dispatch_layout(idx, E, R)
    for key in LAYOUT_KEYS:
        np.testing.assert_array_equal(fz[key].cpu().numpy(), o_lay[key], err_msg=key)
    payload, trailer = split_rows(fz["send_rows"].cpu().numpy(), H)
    o_send = oracle.dispatch(x_bits, o_lay["pos"])
    assert np.array_equal(payload, o_send), "fused payload differs from the oracle"
    assert np.array_equal(trailer, oracle.fused_trailers(fz["epoch"], o_lay["slot_src"])), \
        "fused trailers differ from the oracle"
    out = bits(fz["out"])
    assert_same_bits(out, oracle.combine(o_send, o_lay["pos"], wt), "fused combine")
    if expect_out is not None:
        assert np.array_equal(out, expect_out), "fused round trip differs"
    return o_lay, o_send


@pytest.mark.parametrize("name", wl.ORDER)
def test_fused_matches_oracle(epm, name):
    w = wl.WORKLOADS[name]
    c = Case(w)
    say(f"fused {w.describe()}")
    x = to_dev_bits(c.x)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    fz = epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, want_epoch=True)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    # identity experts: the round trip returns x exactly
    check_fused(epm, fz, c.x, c.idx, c.wt, w.E, w.R, w.H, w.k, expect_out=c.x)
    # and equals the three-launch path bit for bit
    lay = epm.ep_dispatch_layout(idx, w.E, w.R)
    send = epm.ep_dispatch(x, lay["pos"])
    out = epm.ep_combine(send, lay["pos"], wt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fz["out"].view(torch.int16))


@pytest.mark.parametrize("name", wl.ORDER)
def test_fused_signed_weights_match_oracle(epm, name):
    """Weights that are not the routing's (signed, not normalised): the fused
    reduction -- a token's row segments reduced in batches before they are
    stored -- gives the oracle's fp32 chain bit for bit, and the three-launch
    combine over the same rows; at H=4096 a row is one short batch."""
    w = wl.WORKLOADS[name]
    c = Case(w)
    rng = np.random.default_rng(w.seed + 77)
    ws = (rng.random(c.wt.shape, dtype=np.float32) * np.float32(1.5) - np.float32(0.5))
    say(f"fused, signed weights, {w.describe()}")
    x = to_dev_bits(c.x)
    idx = torch.from_numpy(c.idx).to(DEV)
    d_ws = torch.from_numpy(ws).to(DEV)
    fz = epm.ep_fused_dispatch_combine(x, idx, d_ws, w.E, w.R, want_epoch=True)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    o_lay = oracle.dispatch_layout(c.idx, w.E, w.R)
    o_send = oracle.dispatch(c.x, o_lay["pos"])
    out = bits(fz["out"])
    if w.T <= 4096:
        assert_same_bits(out, oracle.combine(o_send, o_lay["pos"], ws), "fused, signed weights")
    else:
        toks = np.unique(np.concatenate([np.arange(0, w.T, 7), [w.T - 1]]))
        assert_same_bits(out[toks], oracle.combine_tokens(o_send, o_lay["pos"], ws, toks),
                         "fused, signed weights (sampled tokens)")
    lay = epm.ep_dispatch_layout(idx, w.E, w.R)
    send = epm.ep_dispatch(x, lay["pos"])
    ref = epm.ep_combine(send, lay["pos"], d_ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), fz["out"].view(torch.int16))


def test_fused_epochs_and_reuse(epm):
    """Repeated calls on one workspace: the epoch advances by one per call, and
    a call on new inputs over rows holding the previous call's trailers reads
    only its own rows."""
    w = wl.WORKLOADS["glm45air"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    x1 = to_dev_bits(c.x)
    x2_bits = wl.make_rows(w.T, w.H, seed=4242)
    x2 = to_dev_bits(x2_bits)
    say("fused epochs")
    fz = epm.ep_fused_dispatch_combine(x1, idx, wt, w.E, w.R, want_epoch=True)
    e1 = fz["epoch"]
    for rep in range(6):
        xin, xb = (x2, x2_bits) if rep % 2 == 0 else (x1, c.x)
        fz = epm.ep_fused_dispatch_combine(xin, idx, wt, w.E, w.R, out=fz, want_epoch=True)
        torch.cuda.synchronize()
        assert fz["epoch"] == e1 + rep + 1
        assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
        assert np.array_equal(bits(fz["out"]), xb), f"call {rep}: stale rows were read"
    check_fused(epm, fz, c.x, c.idx, c.wt, w.E, w.R, w.H, w.k, expect_out=c.x)


def test_fused_back_to_back_without_sync(epm):
    w = wl.WORKLOADS["dsv3"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    x = to_dev_bits(c.x)
    say("fused back-to-back x20")
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    for _ in range(20):
        epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    assert np.array_equal(bits(fz["out"]), c.x)


FUSED_EDGE = [
    (1, 8, 1, 1, 1, 11),
    (5, 16, 4, 2, 2, 12),
    (130, 7176, 64, 8, 6, 13),     # ragged rows, runtime-k path
    (8192, 64, 1024, 8, 4, 14),    # 8 scan blocks
    (3000, 520, 33, 3, 5, 15),
    (64, 4096, 128, 16, 64, 16),   # k = 64
    (20000, 256, 16, 4, 8, 17),    # many items, k = 8 path, small rows
    (3, 1 << 20, 4, 2, 2, 18),     # H = 2^20 (maximum): 2 MiB rows, 2048 chunk flags
]


@pytest.mark.parametrize("T,H,E,R,k,seed", FUSED_EDGE)
def test_fused_edge_shapes(epm, T, H, E, R, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = wl.make_rows(T, H, seed)
    o_idx, o_w = oracle.route_topk(logits, k, 1)
    say(f"fused edge T={T} H={H} E={E} R={R} k={k}")
    fz = epm.ep_fused_dispatch_combine(to_dev_bits(x), torch.from_numpy(o_idx).to(DEV),
                                       torch.from_numpy(o_w).to(DEV), E, R, want_epoch=True)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    check_fused(epm, fz, x, o_idx, o_w, E, R, H, k, expect_out=x)


def test_fused_bounded_waits_drain_and_recover(epm):
    """With a spin limit of one polling round, unsatisfied waits give up at
    once: the call ends with EP_OK or EP_ERR_TIMEOUT (never hangs), and the
    next call on the same workspace is correct."""
    w = wl.WORKLOADS["dsv3"]
    c = Case(w)
    idx = torch.from_numpy(c.idx).to(DEV)
    wt = torch.from_numpy(c.wt).to(DEV)
    x = to_dev_bits(c.x)
    say("fused spin_limit=1")
    fz = epm.fused_outputs(w.T, w.H, w.k, w.E, w.R, DEV)
    epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz, spin_limit=1)
    rc = epm.ep_get_device_error(fz["workspace"])
    assert rc in (epm.EP_OK, epm.EP_ERR_TIMEOUT)
    print(f"[gpu-test] spin_limit=1 -> {rc}")
    say("fused after a bounded-wait call")
    epm.ep_fused_dispatch_combine(x, idx, wt, w.E, w.R, out=fz)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
    assert np.array_equal(bits(fz["out"]), c.x)


def test_fused_bad_id_beside_the_batched_path(epm):
    """k = 8 and 14 KiB rows: every token but one takes the batched reduction;
    the token with an id outside [0, E) gets pos = -1 for that pick and the
    segment-at-a-time path, where the missing row counts as zeros.  The call
    reports the device error, equals the three-launch path bit for bit, and
    the bad token's output is the oracle's fp32 chain over its rows with that
    one row zero."""
    T, H, E, R, k = 96, 7168, 64, 8, 8
    rng = np.random.default_rng(23)
    idx, wt = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    wt = (wt - np.float32(0.05)).astype(np.float32)        # not normalised
    bad_t, bad_j = 37, 3
    idx[bad_t, bad_j] = E + 5
    x = wl.make_rows(T, H, 24)
    say("fused, k=8, one bad id")
    d_x, d_idx, d_w = to_dev_bits(x), torch.from_numpy(idx).to(DEV), torch.from_numpy(wt).to(DEV)
    fz = epm.ep_fused_dispatch_combine(d_x, d_idx, d_w, E, R)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_ERR_DEVICE
    pos = fz["pos"].cpu().numpy()
    assert pos[bad_t, bad_j] == -1
    lay = epm.ep_dispatch_layout(d_idx, E, R)
    send = epm.ep_dispatch(d_x, lay["pos"])
    ref = epm.ep_combine(send, lay["pos"], d_w)
    torch.cuda.synchronize()
    assert np.array_equal(lay["pos"].cpu().numpy(), pos)
    out = bits(fz["out"])
    assert np.array_equal(out, bits(ref)), "fused differs from the three-launch path"
    rows = np.stack([x[bad_t] if j != bad_j else np.zeros(H, np.uint16) for j in range(k)])
    want = oracle.combine(rows, np.arange(k, dtype=np.int32).reshape(1, k), wt[bad_t:bad_t + 1])
    assert_same_bits(out[bad_t:bad_t + 1], want, "the token with a bad id")


def test_fused_flags_bad_expert_ids(epm):
    T, H, k, E, R = 300, 64, 2, 8, 2
    rng = np.random.default_rng(21)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[10, 0] = 99
    x = wl.make_rows(T, H, 21)
    wt = np.full((T, k), 0.5, np.float32)
    say("fused with bad ids")
    fz = epm.ep_fused_dispatch_combine(to_dev_bits(x), torch.from_numpy(idx).to(DEV),
                                       torch.from_numpy(wt).to(DEV), E, R)
    torch.cuda.synchronize()
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_ERR_DEVICE
    assert fz["pos"].cpu().numpy()[10, 0] == -1
    # the next good call clears it
    idx[10, 0] = 3
    epm.ep_fused_dispatch_combine(to_dev_bits(x), torch.from_numpy(idx).to(DEV),
                                  torch.from_numpy(wt).to(DEV), E, R, out=fz)
    assert epm.ep_get_device_error(fz["workspace"]) == epm.EP_OK
