"""The fused mode's payload-before-flag order under a weak memory model (CPU).

UBEP sec. 3.4 / Fig. 6 (Data-as-Flag) relies on the data being visible
before its readiness word; UBEP sec. 6 / Table 5: without single-copy atomic
writes of a whole block, that order takes fences or acknowledgements.  On
gfx950 each XCD has its own L2, which is not coherent with the other XCDs for
plain stores, and stores complete out of order.  The emulation's weak memory
mode (tests/emu/fake/hip/hip_runtime.h, tests/emu/emu_runtime.cpp) models
exactly that:
  - each simulated XCD has a private write-back cache; plain stores land dirty
    in it and reach memory only at an agent-scope release or the kernel's end;
  - stores with the agent-coherence bit (sc1) and atomic stores write through
    to memory; coherent and atomic loads read memory;
  - plain loads may return a stale cached copy until an agent-scope acquire
    invalidates the cache;
  - every store completes out of order, at the latest at s_waitcnt vmcnt(0).

Pins of the model itself (message-passing litmus tests): it shows a stale
read for plain data behind a coherent flag and for a missing acquire, and
never for the ordered patterns -- among them one lane's flag behind the
wave's wait for every lane's stores (s_waitcnt counts the wave's stores, not
the lane's).

The real kernels, every readiness mode of the fused kernel included, give the
oracle's answer under the model.  Two negative controls, each a build that
changes one thing in the emulated memory system only, must fail the same
check: sc1 stores treated as plain stores, and s_waitcnt not waiting for
stores.  They run in a subprocess, so a mutant that hangs or crashes cannot
take the test process with it.
"""
import ctypes
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from combine_ep_route_topk_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
EMU = os.path.join(HERE, "emu")


@pytest.fixture(scope="module")
def emu_build():
    sys.path.insert(0, EMU)
    import build
    if build.compiler() is None:
        pytest.skip("clang++ not available")
    return build


@pytest.fixture(scope="module")
def lib(emu_build):
    sys.path.insert(0, EMU)
    import weak_fused
    return weak_fused.load(emu_build.build())


@pytest.mark.parametrize("mode,stale", [(0, "always"), (1, "never"), (2, "never"),
                                        (3, "sometimes"), (4, "never"), (5, "never")])
def test_model_message_passing_litmus(lib, mode, stale):
    lib.emu_set_weak(1, ctypes.c_ulonglong(99))
    try:
        n = lib.emu_litmus_message_passing(mode, 40)
    finally:
        lib.emu_set_weak(0, ctypes.c_ulonglong(0))
    if stale == "always":
        assert n == 40
    elif stale == "never":
        assert n == 0
    else:
        assert n > 0


def test_fused_modes_hold_under_the_weak_model(lib):
    import weak_fused
    calls, bad = weak_fused.run(lib)
    assert calls == len(weak_fused.SHAPES) * len(weak_fused.MODES) * 2
    assert not bad, bad


def _aligned(nbytes, align=256):
    buf = np.zeros(nbytes + align, np.uint8)
    off = (-buf.ctypes.data) % align
    return buf[off:off + nbytes]


@pytest.mark.parametrize("T,H,E,R,k,seed", [(4608, 8, 1024, 8, 8, 9), (600, 64, 256, 32, 8, 5)])
def test_chain_holds_under_the_weak_model(lib, T, H, E, R, k, seed):
    """route -> layout (4608 x 8 slots over 1024 experts: the separate
    look-back scan, whose status words carry their own values) -> dispatch ->
    combine, with the weak model on."""
    p = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    lib.ep_dispatch_layout_workspace_bytes.restype = ctypes.c_size_t
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = _aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    x[:] = wl.make_rows(T, H, seed + 1)
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    lay = {key: np.zeros(n, np.int32) for key, n in
           (("expert_counts", E), ("expert_offsets", E + 1), ("rank_counts", R),
            ("rank_offsets", R + 1), ("pos", T * k), ("slot_src", T * k))}
    ws = _aligned(lib.ep_dispatch_layout_workspace_bytes(T, k, E, R))
    send = _aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    out = _aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    lib.emu_set_weak(1, ctypes.c_ulonglong(seed))
    try:
        assert lib.ep_route_topk(p(logits), T, E, k, 1, p(idx), p(w), None) == 0
        assert lib.ep_dispatch_layout(p(idx), T, k, E, R, *[p(lay[key]) for key in lay], p(ws),
                                      ctypes.c_size_t(ws.size), None) == 0
        assert lib.ep_get_device_error(p(ws), None) == 0
        assert lib.ep_dispatch(p(x), T, H, k, p(lay["pos"]), p(send), None) == 0
        assert lib.ep_combine(p(send), p(lay["pos"]), p(w), T, H, k, p(out), None) == 0
    finally:
        lib.emu_set_weak(0, ctypes.c_ulonglong(0))
    o_idx, o_w = oracle.route_topk(logits, k, 1)
    np.testing.assert_array_equal(idx, o_idx)
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    for key in lay:
        np.testing.assert_array_equal(lay[key].reshape(o_lay[key].shape), o_lay[key], err_msg=key)
    assert np.array_equal(send, oracle.dispatch(x, o_lay["pos"]))
    assert np.array_equal(out, x)


@pytest.mark.parametrize("variant,flag", [("sc1_plain", "-DEMU_MUTATE_SC1_STORES_PLAIN"),
                                          ("no_store_wait", "-DEMU_MUTATE_NO_STORE_WAIT")])
def test_negative_control_breaks_the_fused_mode(emu_build, variant, flag):
    """The same check on a build whose emulated memory system drops one
    guarantee the fused kernel relies on: the payload then reaches the
    combine after its readiness word, and the check fails."""
    path = emu_build.build((flag,), variant)
    r = subprocess.run([sys.executable, os.path.join(EMU, "weak_fused.py"), path],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return                      # crashed or aborted: the break was seen too
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["calls"] > 0
    assert len(res["bad"]) > 0, f"{variant}: the mutation went unnoticed"
