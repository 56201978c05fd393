"""The C-ABI library: it loads, exports every symbol its header declares, sizes
workspaces, and rejects bad arguments synchronously -- all without a GPU (no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_route_topk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def ep():
    from combine_ep_route_topk_amd import ep as mod
    return mod


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ep_route_topk", "ep_dispatch_layout", "ep_dispatch", "ep_combine",
                     "ep_fused_dispatch_combine", "ep_fused_dispatch_combine_sync",
                     "ep_combine_grad", "ep_dispatch_grad", "ep_get_device_error"):
        assert required in names


def test_library_exports_every_declared_symbol(ep):
    lib = ep.library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert ep.ep_abi_version() == 1


def test_status_strings(ep):
    lib = ep.library()
    assert lib.ep_status_string(0) == b"EP_OK"
    assert lib.ep_status_string(6) == b"EP_ERR_TIMEOUT"
    assert lib.ep_status_string(99) == b"EP_ERR_UNKNOWN"


def test_workspace_and_stride_queries(ep):
    lib = ep.library()
    # one 1 KiB header, then 256 B-aligned arrays; a bigger problem needs more
    small = lib.ep_dispatch_layout_workspace_bytes(128, 2, 8, 2)
    big = lib.ep_dispatch_layout_workspace_bytes(16384, 8, 256, 64)
    assert small >= 1024 and small % 256 == 0 and big > small
    assert big >= 4 * 16384 * 8          # holds one rank word per slot
    assert lib.ep_dispatch_layout_workspace_bytes(0, 2, 8, 2) == 0
    assert lib.ep_fused_workspace_bytes(16384, 8, 256, 64) > big
    # payload + 16-byte trailer + chunk flags, rounded up to 1 KiB
    for H in (8, 256, 4096, 7168, 7176):
        chunks = -(-2 * H // 1024)
        assert lib.ep_fused_row_stride_bytes(H) == -(-(2 * H + 16 + 8 * chunks) // 1024) * 1024
    assert lib.ep_fused_row_stride_bytes(7) == 0


FAKE = 0x10000          # aligned, never dereferenced: validation fails first


def call(lib, name, *args):
    f = getattr(lib, name)
    rc = f(*args)
    return rc, lib.ep_last_error().decode()


def test_route_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    rc, msg = call(lib, "ep_route_topk", P(FAKE), 0, 8, 2, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_INVALID_ARG and "T=0" in msg
    rc, _ = call(lib, "ep_route_topk", P(FAKE), 4, 8, 9, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc, _ = call(lib, "ep_route_topk", P(FAKE), 4, 2048, 8, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_UNSUPPORTED
    rc, _ = call(lib, "ep_route_topk", P(FAKE), 4, 256, 65, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_UNSUPPORTED
    rc, msg = call(lib, "ep_route_topk", None, 4, 8, 2, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_INVALID_ARG and "NULL" in msg
    rc, msg = call(lib, "ep_route_topk", P(FAKE + 2), 4, 8, 2, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_INVALID_ARG and "aligned" in msg
    rc, _ = call(lib, "ep_route_topk", P(FAKE), 1 << 28, 8, 8, 1, P(FAKE), P(FAKE), None)
    assert rc == ep.EP_ERR_UNSUPPORTED            # T*k >= 2^30


def test_layout_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    need = lib.ep_dispatch_layout_workspace_bytes(64, 2, 8, 2)
    rc, _ = call(lib, "ep_dispatch_layout", f, 64, 2, 8, 3, f, f, f, f, f, None, f, need, None)
    assert rc == ep.EP_ERR_INVALID_ARG            # E % R != 0
    rc, _ = call(lib, "ep_dispatch_layout", f, 64, 2, 8, 2, f, f, f, f, f, None, f, need - 1, None)
    assert rc == ep.EP_ERR_WORKSPACE
    rc, _ = call(lib, "ep_dispatch_layout", f, 64, 2, 8, 2, f, f, f, f, f, None,
                 P(FAKE + 64), need, None)
    assert rc == ep.EP_ERR_INVALID_ARG            # workspace not 256-byte aligned
    rc, _ = call(lib, "ep_dispatch_layout", f, 64, 2, 8, 2, f, f, None, f, f, None, f, need, None)
    assert rc == ep.EP_ERR_INVALID_ARG


def test_dispatch_combine_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    rc, msg = call(lib, "ep_dispatch", f, 16, 12, 2, f, f, None)
    assert rc == ep.EP_ERR_INVALID_ARG and "H=12" in msg
    rc, _ = call(lib, "ep_dispatch", P(FAKE + 8), 16, 16, 2, f, f, None)
    assert rc == ep.EP_ERR_INVALID_ARG            # x not 16-byte aligned
    rc, _ = call(lib, "ep_combine", f, f, f, 16, 16, 0, f, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc, _ = call(lib, "ep_combine", f, f, f, 16, 16, 2, P(FAKE + 4), None)
    assert rc == ep.EP_ERR_INVALID_ARG            # out not 16-byte aligned
    # T*H >= 2^40 elements is refused before anything is launched
    rc, msg = call(lib, "ep_dispatch", f, 1 << 21, 1 << 19, 1, f, f, None)
    assert rc == ep.EP_ERR_UNSUPPORTED and "T*H" in msg
    rc, msg = call(lib, "ep_combine", f, f, f, 1 << 21, 1 << 19, 1, f, None)
    assert rc == ep.EP_ERR_UNSUPPORTED and "T*H" in msg


def test_fused_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    need = lib.ep_fused_workspace_bytes(64, 2, 8, 2)
    rc, _ = call(lib, "ep_fused_dispatch_combine", f, f, f, 64, 16, 2, 8, 2, f, f, f, f, f,
                 P(FAKE + 16), f, f, need, None)
    assert rc == ep.EP_ERR_INVALID_ARG            # send_rows not 128-byte aligned
    rc, _ = call(lib, "ep_fused_dispatch_combine", f, f, f, 64, 16, 2, 8, 2, f, f, f, f, f,
                 f, f, f, need - 256, None)
    assert rc == ep.EP_ERR_WORKSPACE
    e = ctypes.c_uint64(0)
    rc, _ = call(lib, "ep_fused_last_epoch", None, ctypes.byref(e), None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc, _ = call(lib, "ep_fused_last_epoch", f, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc, _ = call(lib, "ep_fused_workspace_init", f, 16, None)
    assert rc == ep.EP_ERR_WORKSPACE
    for bad in (-1, 5):
        rc, msg = call(lib, "ep_fused_dispatch_combine_sync", f, f, f, 64, 16, 2, 8, 2, f, f, f,
                       f, f, f, f, f, need, 0, bad, None)
        assert rc == ep.EP_ERR_INVALID_ARG and "sync" in msg


def test_backward_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    rc, msg = call(lib, "ep_combine_grad", f, f, f, f, 16, 12, 2, f, f, None)
    assert rc == ep.EP_ERR_INVALID_ARG and "H=12" in msg
    rc, _ = call(lib, "ep_combine_grad", f, f, f, f, 16, 16, 2, f, P(FAKE + 2), None)
    assert rc == ep.EP_ERR_INVALID_ARG            # grad_w not 4-byte aligned
    rc, _ = call(lib, "ep_dispatch_grad", f, f, 16, 16, 0, f, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc, msg = call(lib, "ep_dispatch_grad", f, f, 1 << 21, 1 << 19, 1, f, None)
    assert rc == ep.EP_ERR_UNSUPPORTED and "T*H" in msg


def test_rank_coalesce_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    need = lib.ep_rank_coalesce_workspace_bytes(64, 4, 16, 4)
    assert need >= lib.ep_dispatch_layout_workspace_bytes(64, 4, 4, 4) + 64 * 4 * 4
    assert lib.ep_rank_coalesce_workspace_bytes(0, 4, 16, 4) == 0
    args = lambda T, k, E, R, re=f, nb=need: (f, T, k, E, R, f, f, f, f, f, re, f, nb, None)
    rc, msg = call(lib, "ep_rank_coalesce", *args(64, 4, 16, 3))
    assert rc == ep.EP_ERR_INVALID_ARG and "divide" in msg
    rc, msg = call(lib, "ep_rank_coalesce", *args(64, 4, 130, 1))
    assert rc == ep.EP_ERR_UNSUPPORTED and "64" in msg          # 130 local experts per rank
    rc, _ = call(lib, "ep_rank_coalesce", *args(64, 4, 16, 4, re=P(FAKE + 4)))
    assert rc == ep.EP_ERR_INVALID_ARG                          # row_experts not 8-byte aligned
    rc, _ = call(lib, "ep_rank_coalesce", *args(64, 4, 16, 4, nb=need - 1))
    assert rc == ep.EP_ERR_WORKSPACE


def test_expand_records_validation(ep):
    lib = ep.library()
    P = ctypes.c_void_p
    f = P(FAKE)
    need = lib.ep_expand_records_workspace_bytes(100, 8)
    assert need > 0 and lib.ep_expand_records_workspace_bytes(100, 65) == 0
    args = lambda C, H, L, nb=need, rows=f: (rows, f, C, H, L, f, f, f, f, ctypes.c_int64(64),
                                             f, nb, None)
    assert call(lib, "ep_expand_records", *args(0, 16, 8))[0] == ep.EP_ERR_INVALID_ARG
    assert call(lib, "ep_expand_records", *args(100, 16, 65))[0] == ep.EP_ERR_INVALID_ARG
    assert call(lib, "ep_expand_records", *args(100, 12, 8))[0] == ep.EP_ERR_INVALID_ARG
    assert call(lib, "ep_expand_records", *args(100, 16, 8, rows=P(FAKE + 8)))[0] == \
        ep.EP_ERR_INVALID_ARG                                   # rows not 16-byte aligned
    assert call(lib, "ep_expand_records", *args(100, 16, 8, nb=need - 1))[0] == ep.EP_ERR_WORKSPACE


def test_exchange_waves_host_function(ep):
    """Host-only: the library's cyclic exchange waves equal the oracle's, and
    the page's 4-node permutation schedule (RailWave App. A.6, Table 8)."""
    import json
    import numpy as np
    import oracle
    for N in (1, 2, 3, 4, 8, 13):
        np.testing.assert_array_equal(ep.ep_exchange_waves(N), oracle.exchange_waves(N))
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "railwave_table8.json")))
    np.testing.assert_array_equal(ep.ep_exchange_waves(4), g["schedules"]["Permutation"]["waves"])
    lib = ep.library()
    assert call(lib, "ep_exchange_waves", 0, None)[0] == ep.EP_ERR_INVALID_ARG
    assert call(lib, "ep_exchange_waves", 3, None)[0] == ep.EP_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors(ep):
    import torch
    with pytest.raises(ValueError, match="GPU"):
        ep.ep_route_topk(torch.zeros((4, 8)), 2)


def test_header_is_plain_c_and_host_calls_work(tmp_path):
    """A C99 program compiled against include/ep_route_topk.h (gcc, -pedantic
    -Werror) and linked to the library: the boundary needs no C++ and no
    torch; its host-side entry points (validation, sizes, the LPT scheduler)
    run without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    from combine_ep_route_topk_amd import ep
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(ep.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c_abi", "abi_check.c"),
                    "-L", lib_dir, "-lep_route_topk", "-Wl,-rpath," + lib_dir, "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
