"""The large-batch kernels on the host emulation, against the CPU oracle.

On the GPU, scatters and gathers above a size threshold take other kernels
than small ones: dispatch and the gradient scatter stride a capped grid over
whole-row items of 4-8 vectors per lane (with a ragged last segment where the
row needs one), and combine runs batched.  The sizes that
reach them are too large for the emulation, so these tests use a build of
the library whose threshold is 0: every size takes the large-batch kernels.
With 4 emulated CUs the capped grids are 2-3 workgroups, so every wave loops
over many items.

Checked bit for bit: dispatch (UBEP sec. 2.1), combine and dispatch_grad (the
fp32 chain of HyperParallel-MoE sec. 4.1), and grad_y of the combine backward
(HyperParallel-MoE sec. 2.2, Fig. 2(b)); grad_w within the derived bound.
Each shape also runs with picks outside the buffer and, where T % 4 != 0, a
last token group that is not full.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
from combine_ep_route_topk_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gpu_util as gu  # noqa: E402
from exact_bf16 import plant_tie_products  # noqa: E402

# T, H, E, R, k, seed -- the item shape each reaches in the large-batch build
SHAPES = [
    (37, 3584, 64, 8, 8, 61),     # 448 vectors a row: 7 per lane, batched combine
    (22, 4096, 32, 4, 6, 62),     # 512: 8 per lane
    (13, 2048, 16, 4, 4, 63),     # 256: 4 per lane
    (9, 6144, 16, 4, 2, 64),      # 768: 8 per lane and a ragged last segment
    (6, 3584, 16, 4, 3, 65),      # 7 per lane, k = 3 (no compile-time pick count)
    (10, 7176, 64, 8, 8, 66),     # 897 vectors: 8 per lane, ragged; per-wave combine
    (11, 520, 16, 4, 5, 67),      # 65 vectors: one per lane
]


@pytest.fixture(scope="module")
def lib():
    sys.path.insert(0, os.path.join(HERE, "emu"))
    import build as emu_build
    if emu_build.compiler() is None:
        pytest.skip("clang++ not available")
    L = ctypes.CDLL(emu_build.build(("-DEP_SMALL_SCATTER_BYTES=0",), "large_batch"))
    L.ep_last_error.restype = ctypes.c_char_p
    L.emu_set_pool(4)
    return L


def p(a):
    return ctypes.c_void_p(a.ctypes.data)


def aligned(shape, dtype, fill=0):
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    buf = np.zeros(n + 256, np.uint8)
    off = (-buf.ctypes.data) % 256
    a = buf[off:off + n].view(dtype).reshape(shape)
    a[...] = fill
    return a


def inputs(T, H, E, R, k, seed):
    rng = np.random.default_rng(seed)
    idx, w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    pos = oracle.dispatch_layout(idx, E, R)["pos"]
    w = (w - np.float32(0.3)).astype(np.float32)            # signed weights
    x = aligned((T, H), np.uint16)
    x[:] = wl.make_rows(T, H, seed + 1)
    return pos, w, x


def with_lost_picks(pos, T, k):
    """pos with three picks moved outside [0, T*k) (-1, T*k, T*k + 9);
    returns (pos_bad, the rows those picks had)."""
    bad = pos.copy()
    cells = sorted({(0, k - 1), (T // 2, 0), (T - 1, k // 2)})
    lost = [int(pos[t, j]) for t, j in cells]
    for (t, j), v in zip(cells, (-1, T * k, T * k + 9)):
        bad[t, j] = v
    return bad, lost


@pytest.mark.parametrize("lose", [False, True])
@pytest.mark.parametrize("T,H,E,R,k,seed", SHAPES)
def test_large_batch_dispatch_and_combine(lib, T, H, E, R, k, seed, lose):
    pos, w, x = inputs(T, H, E, R, k, seed)
    use, lost = with_lost_picks(pos, T, k) if lose else (pos, [])
    d_pos = aligned(pos.shape, np.int32)
    d_pos[:] = use
    send = aligned((T * k, H), np.uint16, 0xFFFF)
    assert lib.ep_dispatch(p(x), T, H, k, p(d_pos), p(send), None) == 0, lib.ep_last_error()
    ref = oracle.dispatch(x, pos)
    ref[lost] = 0xFFFF
    assert np.array_equal(send, ref), "dispatch"

    y = aligned((T * k, H), np.uint16)
    y[:] = wl.make_rows(T * k, H, seed + 2)
    d_w = aligned(w.shape, np.float32)
    d_w[:] = w
    out = aligned((T, H), np.uint16, 0xFFFF)
    assert lib.ep_combine(p(y), p(d_pos), p(d_w), T, H, k, p(out), None) == 0
    y0 = y.copy()
    y0[lost] = 0
    gu.assert_same_bits(out, oracle.combine(y0, pos, w), "combine")

    gx = aligned((T, H), np.uint16, 0xFFFF)
    assert lib.ep_dispatch_grad(p(y), p(d_pos), T, H, k, p(gx), None) == 0
    gu.assert_same_bits(gx, oracle.dispatch_grad(y0, pos), "dispatch_grad")


@pytest.mark.parametrize("lose", [False, True])
@pytest.mark.parametrize("T,H,E,R,k,seed", SHAPES)
def test_large_batch_combine_grad(lib, T, H, E, R, k, seed, lose):
    pos, w, g = inputs(T, H, E, R, k, seed)
    plant_tie_products(w, g, range(0, T, 2), seed)          # f32 products on bf16 ties
    g[::2, H // 2 + 3] = g[::2, 0]                          # the same tie in other lanes
    g[::2, H - 1] = g[::2, 0]                               # and row segments
    use, lost = with_lost_picks(pos, T, k) if lose else (pos, [])
    d_pos = aligned(pos.shape, np.int32)
    d_pos[:] = use
    d_w = aligned(w.shape, np.float32)
    d_w[:] = w
    y = aligned((T * k, H), np.uint16)
    y[:] = wl.make_rows(T * k, H, seed + 3)
    gy = aligned((T * k, H), np.uint16, 0xFFFF)
    gw = aligned((T, k), np.float32, np.nan)
    rc = lib.ep_combine_grad(p(g), p(y), p(d_pos), p(d_w), T, H, k, p(gy), p(gw), None)
    assert rc == 0, lib.ep_last_error()
    r_gy, r_gw = oracle.combine_grad(g, y, pos, w)
    keep = np.setdiff1d(np.arange(T * k), lost)
    assert np.array_equal(gy[keep], r_gy[keep]), "grad_y"
    assert np.all(gy[lost] == 0xFFFF), "a row outside the buffer's picks was written"
    mask = np.ones((T, k), bool)
    for t, j in zip(*np.nonzero(use != pos)):
        mask[t, j] = False
        assert gw[t, j] == 0.0
    gu.check_grad_w(np.where(mask, gw, 0.0), np.where(mask, r_gw, 0.0), g, y, pos)
