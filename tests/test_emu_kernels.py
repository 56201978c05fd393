"""The library's kernel sources run on the CPU under a host emulation of the
HIP device API (tests/emu), checked against the CPU oracle.

This covers the fused flag-in-payload mode with the same source the GPU runs:
the persistent ticket loop, the epoch-tagged look-back and base words, the
per-row trailers, the bounded waits, and the last-workgroup reset of the
workspace -- with only a handful of workgroups resident at a time, which
exercises the forward-progress argument (an item only waits for smaller
tickets).  Each lane is one thread of the source program here, so these tests
check the program's logic, not how the compiler maps divergent control flow
onto a wave.  The unfused kernels run too, as a check of the emulation itself
against the results the GPU gives.
"""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle
from combine_ep_route_topk_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def emu():
    import sys
    sys.path.insert(0, os.path.join(HERE, "emu"))
    import build as emu_build
    if emu_build.compiler() is None:
        pytest.skip("clang++ not available")
    L = ctypes.CDLL(emu_build.build())
    L.ep_dispatch_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_fused_workspace_bytes.restype = ctypes.c_size_t
    L.ep_fused_row_stride_bytes.restype = ctypes.c_size_t
    L.ep_last_error.restype = ctypes.c_char_p
    L.emu_set_pool(4)
    return L


def p(a):
    return ctypes.c_void_p(a.ctypes.data)


def aligned(nbytes, align=256):
    buf = np.zeros(nbytes + align, np.uint8)
    off = (-buf.ctypes.data) % align
    return buf[off:off + nbytes]


class Emu:
    def __init__(self, L, T, H, E, R, k):
        self.L, self.T, self.H, self.E, self.R, self.k = L, T, H, E, R, k

    def check(self, rc):
        assert rc == 0, self.L.ep_last_error().decode()

    def layout_arrays(self):
        E, R, T, k = self.E, self.R, self.T, self.k
        return dict(expert_counts=np.zeros(E, np.int32), expert_offsets=np.zeros(E + 1, np.int32),
                    rank_counts=np.zeros(R, np.int32), rank_offsets=np.zeros(R + 1, np.int32),
                    pos=np.zeros((T, k), np.int32))

    def unfused(self, logits, x):
        L, T, H, E, R, k = self.L, self.T, self.H, self.E, self.R, self.k
        idx = np.zeros((T, k), np.int32)
        wt = np.zeros((T, k), np.float32)
        self.check(L.ep_route_topk(p(logits), T, E, k, 1, p(idx), p(wt), None))
        lay = self.layout_arrays()
        lay["slot_src"] = np.zeros(T * k, np.int32)
        ws = aligned(L.ep_dispatch_layout_workspace_bytes(T, k, E, R))
        self.check(L.ep_dispatch_layout(p(idx), T, k, E, R, p(lay["expert_counts"]),
                                        p(lay["expert_offsets"]), p(lay["rank_counts"]),
                                        p(lay["rank_offsets"]), p(lay["pos"]), p(lay["slot_src"]),
                                        p(ws), ctypes.c_size_t(ws.size), None))
        xa = aligned(x.nbytes, 16).view(np.uint16).reshape(x.shape)
        xa[:] = x
        send = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
        self.check(L.ep_dispatch(p(xa), T, H, k, p(lay["pos"]), p(send), None))
        out = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
        self.check(L.ep_combine(p(send), p(lay["pos"]), p(wt), T, H, k, p(out), None))
        return idx, wt, lay, send, out

    def fused_setup(self):
        L = self.L
        self.ws = aligned(L.ep_fused_workspace_bytes(self.T, self.k, self.E, self.R))
        self.check(L.ep_fused_workspace_init(p(self.ws), ctypes.c_size_t(self.ws.size), None))
        self.stride = L.ep_fused_row_stride_bytes(self.H)
        self.rows = aligned(self.T * self.k * self.stride, 128).reshape(self.T * self.k, self.stride)
        self.flay = self.layout_arrays()
        self.out = aligned(self.T * self.H * 2, 16).view(np.uint16).reshape(self.T, self.H)

    def fused(self, x, idx, wt, spin_limit=1 << 26, sync=0):
        L = self.L
        xa = aligned(x.nbytes, 16).view(np.uint16).reshape(x.shape)
        xa[:] = x
        e = ctypes.c_uint64(0)
        lay = self.flay
        rc = L.ep_fused_dispatch_combine_sync(
            p(xa), p(np.ascontiguousarray(idx)), p(np.ascontiguousarray(wt)), self.T, self.H,
            self.k, self.E, self.R, p(lay["expert_counts"]), p(lay["expert_offsets"]),
            p(lay["rank_counts"]), p(lay["rank_offsets"]), p(lay["pos"]), p(self.rows),
            p(self.out), p(self.ws), ctypes.c_size_t(self.ws.size),
            ctypes.c_uint32(spin_limit), ctypes.c_int32(sync), None)
        self.check(rc)
        self.check(L.ep_fused_last_epoch(p(self.ws), ctypes.byref(e), None))
        return e.value, L.ep_get_device_error(p(self.ws), None)


SHAPES = [
    # T, H, E, R, k, seed
    (128, 256, 8, 2, 2, 1001),      # the tiny workload's shape
    (128, 7168, 256, 32, 8, 1002),  # the decode-like workload's shape (k = 8 path)
    (5, 16, 4, 2, 2, 3),
    (130, 7176, 64, 8, 6, 4),       # ragged rows, runtime-k path
    (600, 64, 256, 32, 8, 5),       # five layout tiles
    (1, 8, 1, 1, 1, 6),
    (3000, 24, 33, 3, 5, 7),        # fifteen tiles, odd E
    (2560, 16, 1024, 8, 8, 8),      # 20480 counters: bases in the positions launch; fused: three scan items
    (4608, 8, 1024, 8, 8, 9),       # 36864 counters: separate scan launch with look-back; fused: five
    # fewer scatter items than the emulation's 8 workgroups: the fused mode
    # splits the rows into parts (3 parts of 7 chunks; 4 parts of 15, ragged)
    (6, 3584, 16, 4, 8, 10),
    (3, 7176, 64, 8, 6, 11),
]


@pytest.mark.parametrize("T,H,E,R,k,seed", SHAPES)
def test_emulated_kernels_match_oracle(emu, T, H, E, R, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    x = wl.make_rows(T, H, seed)
    o_idx, o_w = oracle.route_topk(logits, k, 1)
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    o_send = oracle.dispatch(x, o_lay["pos"])
    m = Emu(emu, T, H, E, R, k)

    # unfused chain (the emulation reproduces what the GPU computes)
    idx, wt, lay, send, out = m.unfused(logits, x)
    np.testing.assert_array_equal(idx, o_idx)
    np.testing.assert_allclose(wt, o_w, rtol=(k + 4 + 8) * 2.0 ** -24)
    for key in lay:
        np.testing.assert_array_equal(lay[key], o_lay[key], err_msg=key)
    assert np.array_equal(send, o_send)
    assert np.array_equal(out, x)

    # fused: two calls on one workspace, the second on different rows
    m.fused_setup()
    x2 = wl.make_rows(T, H, seed + 1)
    e1, st1 = m.fused(x2, o_idx, o_w)
    assert st1 == 0 and np.array_equal(m.out, x2)
    e2, st2 = m.fused(x, o_idx, o_w)
    assert st2 == 0
    assert e2 == e1 + 1 or (e1 + 1) % (1 << 32) == 0
    for key in m.flay:
        np.testing.assert_array_equal(m.flay[key], o_lay[key], err_msg=key)
    payload = m.rows[:, :2 * H].copy().view(np.uint16)
    assert np.array_equal(payload, o_send), "fused payload"
    assert np.array_equal(m.rows[:, 2 * H:2 * H + 16],
                          oracle.fused_trailers(e2, o_lay["slot_src"])), "fused trailers"
    assert np.array_equal(m.out, x), "fused combine"


@pytest.mark.parametrize("T,H", [(200, 520), (64, 3584), (40, 7176), (40, 8192), (24, 4096),
                                 (6, 3584), (3, 7176), (13, 8192)])
def test_emulated_fused_random_experts_equals_combine(emu, T, H):
    """Non-uniform weights: the fused reduction is bit-identical to ep_combine
    over the same rows (they share the arithmetic) and to the oracle's fp32
    chain.  Rows of 1, 7, 14 (plus a partial segment) and 16 whole 64-vector
    segments: one full batch of 14 segments, a short batch, and both.  The
    scatter side copies a row in runs of 7, 4 and 1 chunks: one wave per row in
    4-token items (rows of at most 8 KiB, and batches of few items; H=4096: 7+1,
    3584: 7), else two waves per row, each half of its chunks (H=8192: 7+1).  The last
    three batches have fewer scatter items than the emulation's 8
    workgroups, so their rows are split into 3, 4 and 2 parts."""
    E, R, k = 16, 4, 8
    rng = np.random.default_rng(11)
    o_idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    wt = rng.random((T, k), dtype=np.float32) - np.float32(0.3)
    x = wl.make_rows(T, H, 12)
    m = Emu(emu, T, H, E, R, k)
    m.fused_setup()
    _, st = m.fused(x, o_idx, wt)
    assert st == 0
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    o_send = oracle.dispatch(x, o_lay["pos"])
    # reference: the unfused combine kernel over the same rows
    out_ref = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    send = aligned(o_send.nbytes, 16).view(np.uint16).reshape(o_send.shape)
    send[:] = o_send
    m.check(emu.ep_combine(p(send), p(o_lay["pos"]), p(wt), T, H, k, p(out_ref), None))
    assert np.array_equal(m.out, out_ref)
    assert np.array_equal(m.out, oracle.combine(o_send, o_lay["pos"], wt))


def test_emulated_bounded_waits_and_bad_ids(emu):
    T, H, E, R, k = 256, 32, 8, 2, 2
    rng = np.random.default_rng(13)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    x = wl.make_rows(T, H, 14)
    m = Emu(emu, T, H, E, R, k)
    m.fused_setup()
    # a spin limit of one polling round: the call drains with OK or TIMEOUT
    _, st = m.fused(x, o_idx, o_w, spin_limit=1)
    assert st in (0, 6)
    # and the workspace is usable again right away
    _, st = m.fused(x, o_idx, o_w)
    assert st == 0 and np.array_equal(m.out, x)
    # an id outside [0, E) is reported and gets pos = -1
    bad = o_idx.copy()
    bad[7, 1] = E + 3
    _, st = m.fused(x, bad, o_w)
    assert st == 5 and m.flay["pos"][7, 1] == -1
    _, st = m.fused(x, o_idx, o_w)
    assert st == 0


BACKWARD_SHAPES = [
    # T, H, E, R, k, seed
    (5, 16, 4, 2, 2, 21),
    (40, 7176, 64, 8, 8, 22),     # ragged last segment, k = 8 path
    (33, 520, 16, 4, 3, 23),      # runtime-k path
    (7, 8, 4, 2, 1, 24),          # one vector per row
    (30, 1032, 16, 4, 4, 25),     # k = 4 path, ragged last segment
    (24, 512, 16, 4, 6, 26),      # k = 6 path
    (20, 520, 16, 4, 5, 27),      # runtime-k path, 5 picks
]


@pytest.mark.parametrize("T,H,E,R,k,seed", BACKWARD_SHAPES)
def test_emulated_backward_matches_oracle(emu, T, H, E, R, k, seed):
    """Backward of combine and of dispatch (HyperParallel-MoE sec. 2.2,
    Fig. 2(b)) on the emulated kernels against the oracle."""
    import gpu_util as gu
    from exact_bf16 import plant_tie_products
    rng = np.random.default_rng(seed)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    pos = oracle.dispatch_layout(o_idx, E, R)["pos"]
    g = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    g[:] = wl.make_rows(T, H, seed + 100)
    plant_tie_products(o_w, g, range(0, T, 2), seed)   # f32 product on a bf16 tie
    y = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    y[:] = wl.make_rows(T * k, H, seed + 200)
    gy = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    gw = np.zeros((T, k), np.float32)
    rc = emu.ep_combine_grad(p(g), p(y), p(pos), p(o_w), T, H, k, p(gy), p(gw), None)
    assert rc == 0, emu.ep_last_error().decode()
    r_gy, r_gw = oracle.combine_grad(g, y, pos, o_w)
    assert np.array_equal(gy, r_gy), "grad_y"
    gu.check_grad_w(gw, r_gw, g, y, pos)

    gx = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    rc = emu.ep_dispatch_grad(p(y), p(pos), T, H, k, p(gx), None)
    assert rc == 0, emu.ep_last_error().decode()
    gu.assert_same_bits(gx, oracle.dispatch_grad(y, pos), "dispatch_grad")


SYNC_NAMES = {0: "item events", 1: "row flags", 2: "checksum", 3: "sentinel", 4: "chunk flags"}


@pytest.mark.parametrize("sync", [1, 2, 3, 4])
@pytest.mark.parametrize("T,H,E,R,k,seed", [(128, 256, 8, 2, 2, 41), (130, 7176, 64, 8, 6, 42),
                                             (600, 64, 256, 32, 8, 43), (5, 16, 4, 2, 2, 44)])
def test_emulated_fused_sync_modes(emu, sync, T, H, E, R, k, seed):
    """The Data-as-Flag variants of the fused mode (UBEP sec. 3.4, Fig. 6):
    row flags, a per-batch checksum, sentinel polling.  Layout, payload and
    combined output match the oracle on two calls in a row, then the default
    mode runs on the same workspace."""
    rng = np.random.default_rng(seed)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    x = wl.make_rows(T, H, seed + 1)
    x2 = wl.make_rows(T, H, seed + 2)
    o_send = oracle.dispatch(x, o_lay["pos"])
    m = Emu(emu, T, H, E, R, k)
    m.fused_setup()
    for xi in (x2, x):
        _, st = m.fused(xi, o_idx, o_w, sync=sync)
        assert st == 0, SYNC_NAMES[sync]
        assert np.array_equal(m.out, oracle.combine(oracle.dispatch(xi, o_lay["pos"]),
                                                    o_lay["pos"], o_w)), SYNC_NAMES[sync]
    for key in m.flay:
        np.testing.assert_array_equal(m.flay[key], o_lay[key], err_msg=key)
    payload = m.rows[:, :2 * H].copy().view(np.uint16)
    assert np.array_equal(payload, o_send), "payload"
    _, st = m.fused(x2, o_idx, o_w, sync=0)
    assert st == 0
    assert np.array_equal(m.out, oracle.combine(oracle.dispatch(x2, o_lay["pos"]), o_lay["pos"], o_w))


def test_emulated_sentinel_collision_is_reported(emu):
    """A token whose leading 16 bytes hold the reserved pattern cannot be told
    from an unwritten row: the call reports it (EP_ERR_DEVICE) instead of
    waiting, and the workspace works again on the next call."""
    T, H, E, R, k = 64, 32, 8, 2, 2
    rng = np.random.default_rng(51)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    x = wl.make_rows(T, H, 52)
    bad = x.copy()
    bad[9, 2:4] = 0x7FA5                  # one 32-bit word of the reserved pattern
    m = Emu(emu, T, H, E, R, k)
    m.fused_setup()
    _, st = m.fused(bad, o_idx, o_w, sync=3)
    assert st == 5
    assert b"sentinel" in emu.ep_last_error()
    _, st = m.fused(x, o_idx, o_w, sync=3)
    assert st == 0
    o_lay = oracle.dispatch_layout(o_idx, E, R)
    assert np.array_equal(m.out, oracle.combine(oracle.dispatch(x, o_lay["pos"]),
                                                o_lay["pos"], o_w))
    # the same rows through the other modes are fine: the pattern is reserved
    # only in the sentinel mode
    for sync in (0, 1, 2, 4):
        _, st = m.fused(bad, o_idx, o_w, sync=sync)
        assert st == 0


@pytest.mark.parametrize("seed", range(4))
def test_emulated_slices_and_window_copy(emu, seed):
    """UBEP sec. 3.3 slices from the emulated search kernel equal the oracle's;
    the window-copy consumer copies every row once, following slices or task
    lists, and skips (and counts) a task outside the buffer."""
    rng = np.random.default_rng(900 + seed)
    E = int(rng.integers(1, 700))
    counts = rng.integers(0, 9, size=E)
    counts[rng.random(E) < 0.4] = 0
    eo = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(eo[-1])
    for P in (1, 5, 64, 130, S + 3):
        start = np.zeros(P + 1, np.int64)
        expert = np.zeros(P, np.int32)
        offset = np.zeros(P, np.int64)
        rc = emu.ep_expert_slices(p(eo), E, P, p(start), p(expert), p(offset), None)
        assert rc == 0, emu.ep_last_error().decode()
        o_start, o_expert, o_offset = oracle.slices(eo, P)
        assert np.array_equal(start, o_start) and np.array_equal(expert, o_expert)
        assert np.array_equal(offset, o_offset)
    # the consumer, on S rows of 48 bytes
    row_bytes = 48
    src = aligned(S * row_bytes + 16, 16)[:max(S * row_bytes, 16)]
    src[:] = rng.integers(0, 256, size=src.size, dtype=np.uint8)
    C = 6
    start, _, _ = oracle.slices(eo, C)
    dst = aligned(src.size, 16)
    bad = np.zeros(1, np.uint32)
    rc = emu.ep_window_copy(p(src), p(dst), ctypes.c_int64(row_bytes), ctypes.c_int64(S), None,
                            None, p(start), C, None, p(bad), None)
    assert rc == 0 and bad[0] == 0
    assert np.array_equal(dst[:S * row_bytes], src[:S * row_bytes])
    # task lists: rows in pieces of 5 over 3 cores, plus one task past the end
    rows = [(r, min(5, S - r)) for r in range(0, S, 5)] + [(S, 2)]
    tasks = np.zeros(len(rows), dtype=[("peer", "<i4"), ("stripe", "<i4"), ("first_row", "<i8"),
                                       ("rows", "<i8"), ("cost", "<f8")])
    tasks["first_row"] = [r for r, _ in rows]
    tasks["rows"] = [n for _, n in rows]
    core_begin = np.array([0, len(rows) // 3, 2 * len(rows) // 3, len(rows)], np.int64)
    dst[:] = 0
    clock = np.zeros(6, np.uint64)
    rc = emu.ep_window_copy(p(src), p(dst), ctypes.c_int64(row_bytes), ctypes.c_int64(S),
                            p(tasks), p(core_begin), None, 3, p(clock), p(bad), None)
    assert rc == 0 and bad[0] == 1
    assert np.array_equal(dst[:S * row_bytes], src[:S * row_bytes])
    assert np.all(clock[1::2] >= clock[0::2])


BATCHED = [
    # T, H, E, R, k, grid, seed: one full batch, then a partial one
    (300, 512, 64, 8, 8, 2, 1101),      # k = 8 path: 300 items, 224 per batch
    (97, 1024, 32, 4, 6, 1, 1102),      # k = 6 path: 194 items, 112 per batch
    (40, 1536, 16, 4, 3, 1, 1103),      # runtime k: 120 items, one full batch and 8 more
    (150, 1024, 32, 8, 4, 1, 1104),     # k = 4 path: 300 items
    (130, 512, 16, 4, 2, 1, 1105),      # k = 2 path: 130 items
    (60, 1024, 32, 4, 5, 1, 1106),      # runtime k: 5 picks, one group of 4 and one of 1
]


def batched(emu, y, pos, w, T, H, k, grid):
    out = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    out[:] = 0xFFFF
    emu.emu_combine_batched.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + \
        [ctypes.c_void_p, ctypes.c_int]
    rc = emu.emu_combine_batched(p(y), p(pos), None if w is None else p(w), T, H, k, p(out), grid)
    assert rc == 0 and emu.emu_errors() == 0
    return out


def unbatched(emu, y, pos, w, T, H, k):
    """The one-item-per-wave kernels (ep_combine / ep_dispatch_grad at these
    small sizes): the same f32 arithmetic, so the same bits."""
    out = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    if w is None:
        rc = emu.ep_dispatch_grad(p(y), p(pos), T, H, k, p(out), None)
    else:
        rc = emu.ep_combine(p(y), p(pos), p(w), T, H, k, p(out), None)
    assert rc == 0, emu.ep_last_error().decode()
    return out


def batched_inputs(T, H, E, R, k, seed):
    rng = np.random.default_rng(seed)
    o_idx, o_w = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    pos = np.ascontiguousarray(oracle.dispatch_layout(o_idx, E, R)["pos"])
    y = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    y[:] = wl.make_rows(T * k, H, seed + 1)
    return y, pos, np.ascontiguousarray(o_w)


@pytest.mark.parametrize("T,H,E,R,k,grid,seed", BATCHED)
def test_emulated_batched_combine(emu, T, H, E, R, k, grid, seed):
    """The batched combine (a batch's outputs held back and stored together)
    on a tiny grid, so full and partial batches both run: the same bits as
    the one-item-per-wave kernel, weighted and with unit weights (the backward
    of dispatch), and both the oracle's fp32 chain bit for bit."""
    y, pos, w = batched_inputs(T, H, E, R, k, seed)
    out = batched(emu, y, pos, w, T, H, k, grid)
    assert np.array_equal(out, unbatched(emu, y, pos, w, T, H, k))
    assert np.array_equal(out, oracle.combine(y, pos, w))
    out1 = batched(emu, y, pos, None, T, H, k, grid)
    assert np.array_equal(out1, unbatched(emu, y, pos, None, T, H, k))
    assert np.array_equal(out1, oracle.dispatch_grad(y, pos))


def test_emulated_batched_combine_skips_picks_outside(emu):
    """A pick whose pos lies outside [0, T*k) counts as a row of zeros, in a
    batch that is otherwise full (the checked path) and in the partial one."""
    T, H, E, R, k, grid = 200, 512, 64, 8, 8, 1
    y, pos, w = batched_inputs(T, H, E, R, k, 1111)
    bad = pos.copy()
    lost = [pos[5, 2], pos[150, 7], pos[199, 0]]
    bad[5, 2], bad[150, 7], bad[199, 0] = -1, T * k + 3, T * k
    out = batched(emu, y, bad, w, T, H, k, grid)
    assert np.array_equal(out, unbatched(emu, y, bad, w, T, H, k))
    y0 = y.copy()
    y0[lost] = 0
    assert np.array_equal(out, unbatched(emu, y0, pos, w, T, H, k))
    # H not a multiple of 512: refused
    emu.emu_combine_batched.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + \
        [ctypes.c_void_p, ctypes.c_int]
    assert emu.emu_combine_batched(p(y), p(pos), p(w), T, 256, k, p(out), grid) != 0


COALESCE = [
    # T, E, R, k, seed
    (128, 256, 32, 8, 1201),     # the decode-like shape: one layout tile over R ranks
    (700, 64, 8, 6, 1202),       # five tiles, runtime k
    (300, 16, 16, 4, 1203),      # one expert per rank: the expert layout itself
    (50, 40, 1, 5, 1204),        # one rank: one record per token
    (257, 128, 2, 8, 1205),      # 64 local experts per rank (the mask's full width)
]


def coalesce_emu(L, idx, E, R):
    T, k = idx.shape
    out = dict(rank_counts=np.zeros(R, np.int32), rank_offsets=np.zeros(R + 1, np.int32),
               row_of_pick=np.zeros((T, k), np.int32), send_pos=np.zeros((T, k), np.int32),
               row_src=np.full(T * k, -7, np.int32), row_experts=np.zeros(T * k, np.uint64))
    L.ep_rank_coalesce_workspace_bytes.restype = ctypes.c_size_t
    ws = aligned(L.ep_rank_coalesce_workspace_bytes(T, k, E, R))
    idx = np.ascontiguousarray(idx)
    rc = L.ep_rank_coalesce(p(idx), T, k, E, R, p(out["rank_counts"]), p(out["rank_offsets"]),
                            p(out["row_of_pick"]), p(out["send_pos"]), p(out["row_src"]),
                            p(out["row_experts"]), p(ws), ctypes.c_size_t(ws.size), None)
    assert rc == 0, L.ep_last_error().decode()
    return out, L.ep_get_device_error(p(ws), None)


@pytest.mark.parametrize("T,E,R,k,seed", COALESCE)
def test_emulated_rank_coalesce_matches_oracle(emu, T, E, R, k, seed):
    """RailWave sec. 3.1-3.2 (one send record per token and destination rank):
    the emulated key, layout and rows kernels against the oracle, bit for bit;
    dispatching x with send_pos writes each record's token row."""
    rng = np.random.default_rng(seed)
    idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    got, status = coalesce_emu(emu, idx, E, R)
    assert status == 0
    ref = oracle.rank_coalesce(idx, E, R)
    C = int(ref["rank_offsets"][R])
    for key in ("rank_counts", "rank_offsets", "row_of_pick", "send_pos"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["row_src"][:C], ref["row_src"])
    np.testing.assert_array_equal(got["row_experts"][:C], ref["row_experts"])
    assert np.all(got["row_src"][C:] == -7)            # rows beyond the records untouched
    H = 16
    x = aligned(T * H * 2, 16).view(np.uint16).reshape(T, H)
    x[:] = wl.make_rows(T, H, seed + 1)
    send = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    send[:] = 0xFFFF
    assert emu.ep_dispatch(p(x), T, H, k, p(got["send_pos"]), p(send), None) == 0
    np.testing.assert_array_equal(send[:C], x[ref["row_src"]])
    assert np.all(send[C:] == 0xFFFF)


def test_emulated_rank_coalesce_reports_bad_ids(emu):
    T, E, R, k = 64, 32, 4, 4
    rng = np.random.default_rng(1210)
    idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    bad = idx.copy()
    bad[5, 1], bad[40, 3] = E, -2
    got, status = coalesce_emu(emu, bad, E, R)
    assert status != 0                                  # EP_ERR_DEVICE
    assert got["row_of_pick"][5, 1] == -1 and got["send_pos"][40, 3] == -1
    # the other picks: the records of the routing without the two bad picks
    keep = np.ones((T, k), bool)
    keep[5, 1] = keep[40, 3] = False
    recs = sorted({(int(e) // (E // R), t) for t in range(T) for j, e in enumerate(bad[t]) if keep[t, j]})
    assert int(got["rank_offsets"][R]) == len(recs)
    np.testing.assert_array_equal(got["row_src"][:len(recs)], [t for _, t in recs])


def expand_emu(L_lib, rows, masks, L, recv_rows):
    C, H = rows.shape
    out = dict(expert_counts=np.zeros(L, np.int32), expert_offsets=np.zeros(L + 1, np.int32),
               pos=np.zeros((C, L), np.int32))
    recv = aligned(max(recv_rows, 1) * H * 2, 16).view(np.uint16)[:recv_rows * H].reshape(recv_rows, H)
    recv[:] = 0xFFFF
    L_lib.ep_expand_records_workspace_bytes.restype = ctypes.c_size_t
    ws = aligned(L_lib.ep_expand_records_workspace_bytes(C, L))
    ra = aligned(rows.nbytes, 16).view(np.uint16).reshape(C, H)
    ra[:] = rows
    ma = np.ascontiguousarray(masks, dtype=np.uint64)
    L_lib.ep_expand_records.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int32] * 3 + \
        [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    rc = L_lib.ep_expand_records(p(ra), p(ma), C, H, L, p(out["expert_counts"]),
                                 p(out["expert_offsets"]), p(out["pos"]), p(recv), recv_rows,
                                 p(ws), ws.size, None)
    assert rc == 0, L_lib.ep_last_error().decode()
    return out, recv, L_lib.ep_get_device_error(p(ws), None)


@pytest.mark.parametrize("T,E,R,k,seed", [(300, 64, 8, 6, 1401), (128, 256, 32, 8, 1402),
                                          (90, 128, 2, 8, 1403)])
def test_emulated_expand_records_gives_each_ranks_segment(emu, T, E, R, k, seed):
    """The receiver's side of coalescing: each rank's records, expanded into
    its local experts' slots, equal its segment of the plain dispatch."""
    rng = np.random.default_rng(seed)
    idx, _ = oracle.route_topk(rng.standard_normal((T, E), dtype=np.float32), k, 1)
    H, L = 16, E // R
    x = wl.make_rows(T, H, seed + 1)
    c = oracle.rank_coalesce(idx, E, R)
    lay = oracle.dispatch_layout(idx, E, R)
    send = oracle.dispatch(x, lay["pos"])
    records = x[c["row_src"]]
    for r in range(R):
        a, b = int(c["rank_offsets"][r]), int(c["rank_offsets"][r + 1])
        if a == b:
            continue
        n = int(lay["rank_counts"][r])
        got, recv, status = expand_emu(emu, records[a:b], c["row_experts"][a:b], L, n)
        assert status == 0
        ref = oracle.expand_records(c["row_experts"][a:b], L)
        for key in ("expert_counts", "expert_offsets", "pos"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
        np.testing.assert_array_equal(recv, send[lay["rank_offsets"][r]:lay["rank_offsets"][r + 1]])


def test_emulated_expand_records_reports_overflow_and_stray_bits(emu):
    rows = wl.make_rows(6, 8, 1410)
    masks = np.array([3, 1, 2, 4, 1, 6], np.uint64)        # 9 slots over L = 3
    got, recv, status = expand_emu(emu, rows, masks, 3, 9)
    assert status == 0
    got, recv, status = expand_emu(emu, rows, masks, 3, 7)  # room for 7 of 9 slots
    assert status != 0
    ref = oracle.expand_records(masks, 3)
    full = np.full((9, 8), 0xFFFF, np.uint16)
    for c in range(6):
        for i in range(3):
            if ref["pos"][c, i] >= 0:
                full[ref["pos"][c, i]] = rows[c]
    np.testing.assert_array_equal(recv, full[:7])           # nothing past the buffer
    bad = masks.copy()
    bad[2] |= np.uint64(1 << 3)                             # no local expert 3
    _, _, status = expand_emu(emu, rows, bad, 3, 9)
    assert status != 0


def _chain_cases():
    with open(os.path.join(os.path.dirname(__file__), "golden", "combine_chain.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _chain_cases(), ids=lambda c: c["name"])
def test_emulated_combine_golden_chain_cases(emu, case):
    """The hand-derived fp32-chain cases through the kernels' own source, on
    both combine kernels: each case's values fill every column (H = 512) of
    every token; the one-item-per-wave kernel and the batched one (one
    workgroup) must give the hand-derived pattern everywhere."""
    k, T0, H = case["k"], case["T"], 512
    reps = 4
    T = T0 * reps
    y1 = np.array(case["y"], np.uint16)[:, 0]
    y = aligned(T * k * H * 2, 16).view(np.uint16).reshape(T * k, H)
    y[:] = np.tile(y1, reps)[:, None]
    pos = np.ascontiguousarray(
        (np.tile(np.array(case["pos"], np.int32), (reps, 1))
         + (np.arange(reps)[:, None] * (T0 * k)).repeat(T0, 0)).astype(np.int32))
    w = np.ascontiguousarray(np.tile(np.array(case["w_bits"], np.uint32).view(np.float32),
                                     (reps, 1)))
    want = np.repeat(np.tile(np.array(case["out"], np.uint16), reps)[:, None], H, axis=1)
    assert np.array_equal(unbatched(emu, y, pos, w, T, H, k), want), case["why"]
    assert np.array_equal(batched(emu, y, pos, w, T, H, k, 1), want), case["why"]
