"""ep_dispatch_layout_noalloc: the layout entry point that allocates nothing,
for callers that cannot allocate device memory (graph capture, tight serving
loops).  Its workspace is the library's static scratch array, one per GPU.

Bar: its outputs equal ep_dispatch_layout's (which takes a caller-owned
workspace) bit for bit, on calls in a row whose sizes shrink -- each call
runs on whatever the previous call left in the shared array -- through the C
ABI on the GPU and through the kernels' own source on the CPU.  Sizes past
the scratch's limit are refused before anything runs.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

from combine_ep_route_topk_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
KEYS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos", "slot_src")

# Largest first, so every later call is smaller than the one before it.
#   T, E, R, k, seed
CASES = [
    (16384, 1024, 8, 4, 11),   # 65,536 counters: histogram, look-back scan and positions launches
    (4096, 256, 32, 8, 12),    # the DeepSeek-V3-like shape: histogram + one scan/positions launch
    (3000, 33, 3, 5, 13),      # odd E, ragged last tile
    (128, 256, 32, 8, 14),     # one tile: the single-workgroup kernel
]


def _inputs(T, E, k, seed, bad=False):
    idx, _ = wl.random_topk(T, E, k, seed)
    if bad:                                  # ids outside [0, E) get pos = -1
        idx[T // 2, 0] = E
        idx[T - 1, k - 1] = -3
    return np.ascontiguousarray(idx)


@pytest.mark.gpu
def test_noalloc_layout_equals_the_workspace_layout():
    import torch
    from combine_ep_route_topk_amd import ep
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dev = torch.device("cuda:0")
    for n, (T, E, R, k, seed) in enumerate(CASES):
        for bad in (False, True):
            print(f"[gpu-test] noalloc layout T={T} E={E} R={R} k={k} bad_ids={bad}", flush=True)
            idx = torch.from_numpy(_inputs(T, E, k, seed + n, bad)).to(dev)
            # both output sets start from the same poison: with bad ids the
            # slot_src rows past the counted slots are left as they were
            ref = ep.layout_outputs(T, k, E, R, dev)
            out = ep.layout_outputs(T, k, E, R, dev)
            for key in KEYS:
                ref[key].fill_(-7)
                out[key].fill_(-7)
            ep.ep_dispatch_layout(idx, E, R, out=ref)
            ep.ep_dispatch_layout_noalloc(idx, E, R, out)
            torch.cuda.synchronize()
            for key in KEYS:
                assert torch.equal(out[key], ref[key]), (key, T, E, k, bad)
            assert (ep.ep_get_device_error(ref["workspace"]) == ep.EP_OK) != bad


def test_noalloc_layout_refuses_sizes_past_the_scratch():
    from combine_ep_route_topk_amd import ep
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(0x10000)                            # never dereferenced: validation fails first
    T, k, E, R = 1 << 20, 8, 256, 32
    assert lib.ep_dispatch_layout_workspace_bytes(T, k, E, R) > 16 << 20
    rc = lib.ep_dispatch_layout_noalloc(f, T, k, E, R, f, f, f, f, f, None, None)
    assert rc == ep.EP_ERR_UNSUPPORTED
    assert b"static" in lib.ep_last_error()
    rc = lib.ep_dispatch_layout_noalloc(None, 64, 2, 8, 2, f, f, f, f, f, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG


def _aligned(nbytes, align=256):
    buf = np.zeros(nbytes + align, np.uint8)
    off = (-buf.ctypes.data) % align
    return buf[off:off + nbytes]


def test_emulated_noalloc_layout_equals_the_workspace_layout():
    """The same check on the CPU, through the kernels' own source built for
    the host (the static array is then an ordinary host array)."""
    sys.path.insert(0, os.path.join(HERE, "emu"))
    import build as emu_build
    if emu_build.compiler() is None:
        pytest.skip("clang++ not available")
    L = ctypes.CDLL(emu_build.build())
    L.ep_dispatch_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_last_error.restype = ctypes.c_char_p
    L.emu_set_pool(4)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    for n, (T, E, R, k, seed) in enumerate([(3000, 33, 3, 5, 21), (600, 256, 32, 8, 22),
                                            (128, 8, 2, 2, 23)]):
        idx = _inputs(T, E, k, seed + n, bad=(n == 1))
        res = []
        for noalloc in (False, True):
            o = dict(expert_counts=np.full(E, -7, np.int32),
                     expert_offsets=np.full(E + 1, -7, np.int32),
                     rank_counts=np.full(R, -7, np.int32), rank_offsets=np.full(R + 1, -7, np.int32),
                     pos=np.full((T, k), -7, np.int32), slot_src=np.full(T * k, -7, np.int32))
            args = [p(idx), T, k, E, R] + [p(o[key]) for key in KEYS]
            if noalloc:
                rc = L.ep_dispatch_layout_noalloc(*args, None)
            else:
                ws = _aligned(L.ep_dispatch_layout_workspace_bytes(T, k, E, R))
                rc = L.ep_dispatch_layout(*args, p(ws), ctypes.c_size_t(ws.size), None)
            assert rc == 0, L.ep_last_error().decode()
            res.append(o)
        for key in KEYS:
            np.testing.assert_array_equal(res[1][key], res[0][key], err_msg=key)
