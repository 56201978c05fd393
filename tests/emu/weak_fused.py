"""Runs the fused flag-in-payload mode, in every readiness mode, on the host
emulation with its weak memory mode on, and compares layout, payload and
combined output with the CPU oracle.

Test infrastructure.  Imported by tests/test_emu_weak_memory.py for the real
library, and run as a script (python weak_fused.py LIB) for the negative
controls -- libraries built with a mutation of the emulated memory system --
so that a mutant that crashes or hangs cannot take the test process with it.
The script prints one JSON line: {"calls": n, "bad": [descriptions]}.

UBEP sec. 3.4 and Fig. 6 (Data-as-Flag: the readiness word travels with the
data), sec. 6 and Table 5 (without single-copy atomic writes of a whole
block, ordering needs fences or acknowledgements): the payload must be
visible before its readiness word.
"""
import ctypes
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from combine_ep_route_topk_amd import workloads as wl  # noqa: E402

# T, H, E, R, k, seed (the fourth: k = 8 rows of 7 whole 64-vector segments, which the combine side
# reduces as one batch behind the acquire; the last: 3 scatter items for the emulation's 8
# workgroups, so in item-event mode each row is split into 3 parts with an event word each)
SHAPES = [(128, 256, 8, 2, 2, 1001), (600, 64, 256, 32, 8, 5), (130, 7176, 64, 8, 6, 4),
          (48, 3584, 16, 4, 8, 7), (6, 3584, 16, 4, 8, 8)]
MODES = (0, 1, 2, 3, 4)
SPIN_LIMIT = 4096


def _aligned(nbytes, align=256):
    buf = np.zeros(nbytes + align, np.uint8)
    off = (-buf.ctypes.data) % align
    return buf[off:off + nbytes]


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def load(lib_path):
    L = ctypes.CDLL(lib_path)
    L.ep_fused_workspace_bytes.restype = ctypes.c_size_t
    L.ep_fused_row_stride_bytes.restype = ctypes.c_size_t
    L.ep_last_error.restype = ctypes.c_char_p
    L.emu_set_pool(8)
    return L


def run(L, seed=12345):
    """Two calls per (shape, mode) on one workspace, with different x: the
    second call's rows overwrite the first's.  Returns (calls, bad)."""
    L.emu_set_weak(1, ctypes.c_ulonglong(seed))
    calls, bad = 0, []
    try:
        for T, H, E, R, k, s in SHAPES:
            rng = np.random.default_rng(s)
            idx, w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
            lay = oracle.dispatch_layout(idx, E, R)
            ws = _aligned(L.ep_fused_workspace_bytes(T, k, E, R))
            assert L.ep_fused_workspace_init(_p(ws), ctypes.c_size_t(ws.size), None) == 0
            stride = L.ep_fused_row_stride_bytes(H)
            rows = _aligned(T * k * stride, 128).reshape(T * k, stride)
            out = _aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
            got = {key: np.zeros(n, np.int32) for key, n in
                   (("expert_counts", E), ("expert_offsets", E + 1), ("rank_counts", R),
                    ("rank_offsets", R + 1), ("pos", T * k))}
            for sync in MODES:
                for xs in (s + 1, s + 2):
                    x = _aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
                    x[:] = wl.make_rows(T, H, xs)
                    calls += 1
                    what = f"T={T} H={H} k={k} sync={sync} x={xs}"
                    rc = L.ep_fused_dispatch_combine_sync(
                        _p(x), _p(idx), _p(w), T, H, k, E, R, _p(got["expert_counts"]),
                        _p(got["expert_offsets"]), _p(got["rank_counts"]),
                        _p(got["rank_offsets"]), _p(got["pos"]), _p(rows), _p(out), _p(ws),
                        ctypes.c_size_t(ws.size), ctypes.c_uint32(SPIN_LIMIT),
                        ctypes.c_int32(sync), None)
                    if rc != 0:
                        bad.append(f"{what}: rc={rc} {L.ep_last_error().decode()}")
                        continue
                    st = L.ep_get_device_error(_p(ws), None)
                    send = oracle.dispatch(x, lay["pos"])
                    if st != 0:
                        bad.append(f"{what}: device status {st}")
                    elif any(not np.array_equal(got[key].reshape(lay[key].shape), lay[key])
                             for key in got):
                        bad.append(f"{what}: layout")
                    elif not np.array_equal(rows[:, :2 * H].copy().view(np.uint16), send):
                        bad.append(f"{what}: payload")
                    elif not np.array_equal(out, oracle.combine(send, lay["pos"], w)):
                        bad.append(f"{what}: combined output")
    finally:
        L.emu_set_weak(0, ctypes.c_ulonglong(0))
    return calls, bad


if __name__ == "__main__":
    n, b = run(load(sys.argv[1]))
    print(json.dumps({"calls": n, "bad": b}), flush=True)
