"""Python binding of libep_route_topk (include/ep_route_topk.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors live on the GPU (torch is used for device memory and
streams); bf16 tensors are passed as their raw 16-bit patterns.  Functions
mirror the C entry points of the same name; outputs may be passed in
pre-allocated (the benchmark does) or are allocated here with torch.empty.

Importing this module loads the built library and fails loudly if it is
missing: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as _np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_route_topk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
        "g.build()' or python combine_ep_route_topk_amd/_build.py). "
        "combine_ep_route_topk_amd has no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_sz = ctypes.c_size_t

_SIGS = {
    "ep_abi_version": ([], ctypes.c_int),
    "ep_status_string": ([ctypes.c_int], ctypes.c_char_p),   # ep_status is an int-sized enum
    "ep_last_error": ([], ctypes.c_char_p),
    "ep_route_topk": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P], ctypes.c_int),
    "ep_dispatch_layout_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "ep_dispatch_layout": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _P, _sz, _P],
                           ctypes.c_int),
    "ep_dispatch_layout_noalloc": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _P],
                                   ctypes.c_int),
    "ep_dispatch": ([_P, _i32, _i32, _i32, _P, _P, _P], ctypes.c_int),
    "ep_combine": ([_P, _P, _P, _i32, _i32, _i32, _P, _P], ctypes.c_int),
    "ep_combine_grad": ([_P, _P, _P, _P, _i32, _i32, _i32, _P, _P, _P], ctypes.c_int),
    "ep_dispatch_grad": ([_P, _P, _i32, _i32, _i32, _P, _P], ctypes.c_int),
    "ep_fused_row_stride_bytes": ([_i32], _sz),
    "ep_fused_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "ep_fused_workspace_init": ([_P, _sz, _P], ctypes.c_int),
    "ep_fused_dispatch_combine": ([_P, _P, _P, _i32, _i32, _i32, _i32, _i32, _P, _P, _P, _P,
                                   _P, _P, _P, _P, _sz, _P], ctypes.c_int),
    "ep_fused_dispatch_combine_sync": ([_P, _P, _P, _i32, _i32, _i32, _i32, _i32, _P, _P, _P,
                                        _P, _P, _P, _P, _P, _sz, _u32, _i32, _P],
                                       ctypes.c_int),
    "ep_fused_last_epoch": ([_P, ctypes.POINTER(ctypes.c_uint64), _P], ctypes.c_int),
    "ep_expert_slices": ([_P, _i32, _i32, _P, _P, _P, _P], ctypes.c_int),
    "ep_rank_coalesce_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "ep_rank_coalesce": ([_P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _P, _sz, _P],
                         ctypes.c_int),
    "ep_exchange_waves": ([_i32, _P], ctypes.c_int),
    "ep_expand_records_workspace_bytes": ([_i32, _i32], _sz),
    "ep_expand_records": ([_P, _P, _i32, _i32, _i32, _P, _P, _P, _P, ctypes.c_int64, _P, _sz, _P],
                          ctypes.c_int),
    "ep_lpt_task_count": ([_P, _i32, ctypes.c_int64], ctypes.c_int64),
    "ep_lpt_partition": ([_P, _i32, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P, _i32, _i32,
                          _P, ctypes.c_int64, _P, _P], ctypes.c_int),
    "ep_window_copy": ([_P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _i32, _P, _P, _P],
                       ctypes.c_int),
    "ep_get_device_error": ([_P, _P], ctypes.c_int),
    "ep_set_timing_events": ([_P, _P], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_WORKSPACE = 0, 1, 2, 3
EP_ERR_LAUNCH, EP_ERR_DEVICE, EP_ERR_TIMEOUT = 4, 5, 6
# How the fused mode's combine waits for the rows (ep_fused_sync in the header)
EP_FUSED_SYNC_ITEM_EVENTS, EP_FUSED_SYNC_ROW_FLAG = 0, 1
EP_FUSED_SYNC_CHECKSUM, EP_FUSED_SYNC_SENTINEL, EP_FUSED_SYNC_CHUNK_FLAG = 2, 3, 4


class EpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_lib.ep_status_string(status).decode()}: {detail}")


def _check(rc: int) -> None:
    if rc != EP_OK:
        raise EpError(rc, _lib.ep_last_error().decode())


def library() -> ctypes.CDLL:
    return _lib


def ep_abi_version() -> int:
    return _lib.ep_abi_version()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _bits_ok(t: torch.Tensor, name: str, shape: tuple | None = None):
    """bf16 payloads: torch.bfloat16 (or int16/uint16 holding the bits)."""
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 bit patterns, got {t.dtype}")
    _need(t, name, t.dtype, shape)


# ------------------------------------------------------------------- route
def ep_route_topk(logits: torch.Tensor, k: int, normalize: bool = True,
                  topk_idx: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                  stream=None):
    """logits f32 [T][E] -> (topk_idx i32 [T][k], topk_w f32 [T][k])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k))
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _check(_lib.ep_route_topk(_ptr(logits), T, E, k, int(bool(normalize)), _ptr(topk_idx),
                              _ptr(topk_w), _P(_stream(stream, dev))))
    return topk_idx, topk_w


# ------------------------------------------------------------------- layout
def ep_dispatch_layout_workspace_bytes(T: int, k: int, E: int, R: int) -> int:
    return int(_lib.ep_dispatch_layout_workspace_bytes(T, k, E, R))


def layout_outputs(T: int, k: int, E: int, R: int, device, slot_src: bool = True) -> dict:
    """Allocate the output tensors of ep_dispatch_layout."""
    i32 = dict(dtype=torch.int32, device=device)
    return dict(
        expert_counts=torch.empty(E, **i32), expert_offsets=torch.empty(E + 1, **i32),
        rank_counts=torch.empty(R, **i32), rank_offsets=torch.empty(R + 1, **i32),
        pos=torch.empty((T, k), **i32),
        slot_src=torch.empty(T * k, **i32) if slot_src else None,
        workspace=torch.empty(ep_dispatch_layout_workspace_bytes(T, k, E, R),
                              dtype=torch.uint8, device=device))


def ep_dispatch_layout(topk_idx: torch.Tensor, E: int, R: int, out: dict | None = None,
                       stream=None) -> dict:
    """topk_idx i32 [T][k] -> dict(expert_counts, expert_offsets, rank_counts,
    rank_offsets, pos, slot_src, workspace)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = layout_outputs(T, k, E, R, dev)
    ws = out["workspace"]
    _need(ws, "workspace", torch.uint8)
    for name, shape in (("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                        ("rank_counts", (R,)), ("rank_offsets", (R + 1,)), ("pos", (T, k))):
        _need(out[name], name, torch.int32, shape)
    if out.get("slot_src") is not None:
        _need(out["slot_src"], "slot_src", torch.int32, (T * k,))
    _check(_lib.ep_dispatch_layout(
        _ptr(topk_idx), T, k, E, R, _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["pos"]),
        _ptr(out.get("slot_src")), _ptr(ws), ws.numel(), _P(_stream(stream, dev))))
    return out


def ep_dispatch_layout_noalloc(topk_idx: torch.Tensor, E: int, R: int, out: dict,
                               stream=None) -> dict:
    """ep_dispatch_layout on the library's own static scratch (no workspace,
    nothing allocated by the call): `out` holds the caller's output tensors
    (layout_outputs' keys; 'workspace' is not used)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    for name, shape in (("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                        ("rank_counts", (R,)), ("rank_offsets", (R + 1,)), ("pos", (T, k))):
        _need(out[name], name, torch.int32, shape)
    if out.get("slot_src") is not None:
        _need(out["slot_src"], "slot_src", torch.int32, (T * k,))
    _check(_lib.ep_dispatch_layout_noalloc(
        _ptr(topk_idx), T, k, E, R, _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["pos"]),
        _ptr(out.get("slot_src")), _P(_stream(stream, topk_idx.device))))
    return out


# ------------------------------------------------------------------- dispatch
def ep_dispatch(x: torch.Tensor, pos: torch.Tensor, send: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """x bf16 [T][H], pos i32 [T][k] -> send bf16 [T*k][H]."""
    _bits_ok(x, "x")
    T, H = x.shape
    _need(pos, "pos", torch.int32)
    k = pos.shape[1]
    if pos.shape[0] != T:
        raise ValueError("pos must be [T][k]")
    if send is None:
        send = torch.empty((T * k, H), dtype=x.dtype, device=x.device)
    _bits_ok(send, "send", (T * k, H))
    _check(_lib.ep_dispatch(_ptr(x), T, H, k, _ptr(pos), _ptr(send),
                            _P(_stream(stream, x.device))))
    return send


# ------------------------------------------------------------------- combine
def ep_combine(y: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y bf16 [T*k][H] (send order), pos i32 [T][k], topk_w f32 [T][k] -> out bf16 [T][H]."""
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(y, "y")
    H = y.shape[1]
    if y.shape[0] != T * k:
        raise ValueError("y must have T*k rows")
    _need(topk_w, "topk_w", torch.float32, (T, k))
    if out is None:
        out = torch.empty((T, H), dtype=y.dtype, device=y.device)
    _bits_ok(out, "out", (T, H))
    _check(_lib.ep_combine(_ptr(y), _ptr(pos), _ptr(topk_w), T, H, k, _ptr(out),
                           _P(_stream(stream, y.device))))
    return out


# ------------------------------------------------------------------- backward
def ep_combine_grad(grad_out: torch.Tensor, y: torch.Tensor, pos: torch.Tensor,
                    topk_w: torch.Tensor, grad_y: torch.Tensor | None = None,
                    grad_w: torch.Tensor | None = None, stream=None):
    """grad_out bf16 [T][H], y bf16 [T*k][H], pos i32 [T][k], topk_w f32 [T][k]
    -> (grad_y bf16 [T*k][H], grad_w f32 [T][k])."""
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(grad_out, "grad_out")
    H = grad_out.shape[1]
    if grad_out.shape[0] != T:
        raise ValueError("grad_out must be [T][H]")
    _bits_ok(y, "y", (T * k, H))
    _need(topk_w, "topk_w", torch.float32, (T, k))
    if grad_y is None:
        grad_y = torch.empty((T * k, H), dtype=y.dtype, device=y.device)
    if grad_w is None:
        grad_w = torch.empty((T, k), dtype=torch.float32, device=y.device)
    _bits_ok(grad_y, "grad_y", (T * k, H))
    _need(grad_w, "grad_w", torch.float32, (T, k))
    _check(_lib.ep_combine_grad(_ptr(grad_out), _ptr(y), _ptr(pos), _ptr(topk_w), T, H, k,
                                _ptr(grad_y), _ptr(grad_w), _P(_stream(stream, y.device))))
    return grad_y, grad_w


def ep_dispatch_grad(grad_send: torch.Tensor, pos: torch.Tensor,
                     grad_x: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """grad_send bf16 [T*k][H], pos i32 [T][k] -> grad_x bf16 [T][H]."""
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(grad_send, "grad_send")
    H = grad_send.shape[1]
    if grad_send.shape[0] != T * k:
        raise ValueError("grad_send must have T*k rows")
    if grad_x is None:
        grad_x = torch.empty((T, H), dtype=grad_send.dtype, device=grad_send.device)
    _bits_ok(grad_x, "grad_x", (T, H))
    _check(_lib.ep_dispatch_grad(_ptr(grad_send), _ptr(pos), T, H, k, _ptr(grad_x),
                                 _P(_stream(stream, grad_send.device))))
    return grad_x


# ------------------------------------------------------------------- fused
def ep_fused_row_stride_bytes(H: int) -> int:
    return int(_lib.ep_fused_row_stride_bytes(H))


def ep_fused_workspace_bytes(T: int, k: int, E: int, R: int) -> int:
    return int(_lib.ep_fused_workspace_bytes(T, k, E, R))


def ep_fused_workspace_init(workspace: torch.Tensor, stream=None) -> torch.Tensor:
    _need(workspace, "workspace", torch.uint8)
    _check(_lib.ep_fused_workspace_init(_ptr(workspace), workspace.numel(),
                                        _P(_stream(stream, workspace.device))))
    return workspace


def fused_outputs(T: int, H: int, k: int, E: int, R: int, device) -> dict:
    """Allocate (and initialise the workspace of) ep_fused_dispatch_combine."""
    i32 = dict(dtype=torch.int32, device=device)
    ws = torch.empty(ep_fused_workspace_bytes(T, k, E, R), dtype=torch.uint8, device=device)
    ep_fused_workspace_init(ws)
    return dict(
        expert_counts=torch.empty(E, **i32), expert_offsets=torch.empty(E + 1, **i32),
        rank_counts=torch.empty(R, **i32), rank_offsets=torch.empty(R + 1, **i32),
        pos=torch.empty((T, k), **i32),
        send_rows=torch.empty((T * k, ep_fused_row_stride_bytes(H)), dtype=torch.uint8,
                              device=device),
        out=torch.empty((T, H), dtype=torch.bfloat16, device=device),
        workspace=ws)


def ep_fused_dispatch_combine(x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                              E: int, R: int, out: dict | None = None, spin_limit: int = 0,
                              want_epoch: bool = False, stream=None,
                              sync: int = EP_FUSED_SYNC_ITEM_EVENTS) -> dict:
    """Layout + dispatch + combine (identity experts) in one persistent launch.
    Returns the dict of outputs; with want_epoch the call then synchronises
    and reads back the epoch written into the trailers (key 'epoch').  `sync` picks how combine
    waits for the rows (EP_FUSED_SYNC_*)."""
    _bits_ok(x, "x")
    T, H = x.shape
    _need(topk_idx, "topk_idx", torch.int32)
    k = topk_idx.shape[1]
    _need(topk_w, "topk_w", torch.float32, (T, k))
    if out is None:
        out = fused_outputs(T, H, k, E, R, x.device)
    st = _stream(stream, x.device)
    if sync == EP_FUSED_SYNC_ITEM_EVENTS and not spin_limit:
        _check(_lib.ep_fused_dispatch_combine(
            _ptr(x), _ptr(topk_idx), _ptr(topk_w), T, H, k, E, R, _ptr(out["expert_counts"]),
            _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]),
            _ptr(out["pos"]), _ptr(out["send_rows"]), _ptr(out["out"]),
            _ptr(out["workspace"]), out["workspace"].numel(), _P(st)))
    else:
        _check(_lib.ep_fused_dispatch_combine_sync(
            _ptr(x), _ptr(topk_idx), _ptr(topk_w), T, H, k, E, R, _ptr(out["expert_counts"]),
            _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]),
            _ptr(out["pos"]), _ptr(out["send_rows"]), _ptr(out["out"]),
            _ptr(out["workspace"]), out["workspace"].numel(), int(spin_limit), int(sync),
            _P(st)))
    if want_epoch:
        out["epoch"] = ep_fused_last_epoch(out["workspace"], stream)
    return out


def ep_fused_last_epoch(workspace: torch.Tensor, stream=None) -> int:
    """The epoch the last completed fused call on this workspace wrote into
    its trailers; synchronises the stream first."""
    e = ctypes.c_uint64(0)
    _check(_lib.ep_fused_last_epoch(_ptr(workspace), ctypes.byref(e),
                                    _P(_stream(stream, workspace.device))))
    return int(e.value)


# ------------------------------------------------------------------- partition
# ep_task as a numpy record (host) / raw bytes (device): 32 bytes per task
TASK_DTYPE = _np.dtype([("peer", "<i4"), ("stripe", "<i4"), ("first_row", "<i8"),
                        ("rows", "<i8"), ("cost", "<f8")])


def ep_expert_slices(expert_offsets: torch.Tensor, P: int, out: dict | None = None,
                     stream=None) -> dict:
    """expert_offsets i32 [E+1] (device) -> dict(start i64 [P+1], expert i32 [P],
    offset i64 [P]): P equal contiguous slot slices and their covering experts."""
    _need(expert_offsets, "expert_offsets", torch.int32)
    E = expert_offsets.numel() - 1
    dev = expert_offsets.device
    if out is None:
        out = dict(start=torch.empty(P + 1, dtype=torch.int64, device=dev),
                   expert=torch.empty(P, dtype=torch.int32, device=dev),
                   offset=torch.empty(P, dtype=torch.int64, device=dev))
    _need(out["start"], "start", torch.int64, (P + 1,))
    _need(out["expert"], "expert", torch.int32, (P,))
    _need(out["offset"], "offset", torch.int64, (P,))
    _check(_lib.ep_expert_slices(_ptr(expert_offsets), E, P, _ptr(out["start"]),
                                 _ptr(out["expert"]), _ptr(out["offset"]), _P(_stream(stream, dev))))
    return out


# ------------------------------------------------------------------- coalescing
def coalesce_outputs(T: int, k: int, E: int, R: int, device) -> dict:
    """Allocate the output tensors of ep_rank_coalesce."""
    i32 = dict(dtype=torch.int32, device=device)
    return dict(
        rank_counts=torch.empty(R, **i32), rank_offsets=torch.empty(R + 1, **i32),
        row_of_pick=torch.empty((T, k), **i32), send_pos=torch.empty((T, k), **i32),
        row_src=torch.empty(T * k, **i32),
        row_experts=torch.empty(T * k, dtype=torch.int64, device=device),
        workspace=torch.empty(int(_lib.ep_rank_coalesce_workspace_bytes(T, k, E, R)),
                              dtype=torch.uint8, device=device))


def ep_rank_coalesce(topk_idx: torch.Tensor, E: int, R: int, out: dict | None = None,
                     stream=None) -> dict:
    """topk_idx i32 [T][k] -> dict(rank_counts, rank_offsets, row_of_pick,
    send_pos, row_src, row_experts (u64 bit masks in an int64 tensor),
    workspace): one send record per (token, destination rank).  The number of
    records is rank_offsets[R]; row_src and row_experts are valid below it."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = coalesce_outputs(T, k, E, R, dev)
    ws = out["workspace"]
    _need(ws, "workspace", torch.uint8)
    for name, shape in (("rank_counts", (R,)), ("rank_offsets", (R + 1,)),
                        ("row_of_pick", (T, k)), ("send_pos", (T, k)), ("row_src", (T * k,))):
        _need(out[name], name, torch.int32, shape)
    _need(out["row_experts"], "row_experts", torch.int64, (T * k,))
    _check(_lib.ep_rank_coalesce(
        _ptr(topk_idx), T, k, E, R, _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]),
        _ptr(out["row_of_pick"]), _ptr(out["send_pos"]), _ptr(out["row_src"]),
        _ptr(out["row_experts"]), _ptr(ws), ws.numel(), _P(_stream(stream, dev))))
    return out


def ep_expand_records(rows: torch.Tensor, masks: torch.Tensor, L: int, recv_rows: int,
                      out: dict | None = None, stream=None) -> dict:
    """rows bf16 [C][H] (one rank's records), masks int64 [C] (u64 bit masks
    of local experts) -> dict(expert_counts i32 [L], expert_offsets i32 [L+1],
    pos i32 [C][L], recv bf16 [recv_rows][H], workspace): the records expanded
    into the rank's local experts' slots."""
    _bits_ok(rows, "rows")
    C, H = rows.shape
    _need(masks, "masks", torch.int64, (C,))
    dev = rows.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(expert_counts=torch.empty(L, **i32), expert_offsets=torch.empty(L + 1, **i32),
                   pos=torch.empty((C, L), **i32),
                   recv=torch.empty((recv_rows, H), dtype=rows.dtype, device=dev),
                   workspace=torch.empty(int(_lib.ep_expand_records_workspace_bytes(C, L)),
                                         dtype=torch.uint8, device=dev))
    _need(out["expert_counts"], "expert_counts", torch.int32, (L,))
    _need(out["expert_offsets"], "expert_offsets", torch.int32, (L + 1,))
    _need(out["pos"], "pos", torch.int32, (C, L))
    _bits_ok(out["recv"], "recv", (recv_rows, H))
    ws = out["workspace"]
    _need(ws, "workspace", torch.uint8)
    _check(_lib.ep_expand_records(
        _ptr(rows), _ptr(masks), C, H, L, _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["pos"]), _ptr(out["recv"]), recv_rows, _ptr(ws), ws.numel(),
        _P(_stream(stream, dev))))
    return out


def ep_exchange_waves(N: int):
    """HOST: the cyclic exchange waves -> numpy int32 [N-1][N], peer[w-1][s] =
    (s + w) mod N."""
    peer = _np.zeros((max(N - 1, 0), max(N, 1)), _np.int32)
    _check(_lib.ep_exchange_waves(int(N), peer.ctypes.data if peer.size else None))
    return peer[:, :N]


def ep_lpt_partition(rank_offsets, row_bytes: int, unit_rows: int, C: int, alpha=(0.0,),
                     beta=(1.0,), cap=(1,), tier_of_peer=None):
    """HOST scheduler.  rank_offsets: host int32 [R+1] (numpy or CPU tensor).
    Returns (tasks: numpy TASK_DTYPE [U] grouped by core in stripe order,
    core_begin: int64 [C+1], core_load: float64 [C])."""
    ro = _np.ascontiguousarray(_np.asarray(rank_offsets, dtype=_np.int32))
    R = ro.size - 1
    alpha = _np.ascontiguousarray(alpha, dtype=_np.float64)
    beta = _np.ascontiguousarray(beta, dtype=_np.float64)
    cap = _np.ascontiguousarray(cap, dtype=_np.int32)
    tier = None if tier_of_peer is None else _np.ascontiguousarray(tier_of_peer, dtype=_np.int32)
    n = int(_lib.ep_lpt_task_count(_P(ro.ctypes.data), R, unit_rows))
    if n < 0:
        raise ValueError("bad rank_offsets or unit_rows")
    tasks = _np.zeros(max(n, 1), TASK_DTYPE)
    core_begin = _np.zeros(C + 1, _np.int64)
    load = _np.zeros(C, _np.float64)
    _check(_lib.ep_lpt_partition(
        _P(ro.ctypes.data), R, row_bytes, unit_rows,
        _P(tier.ctypes.data) if tier is not None else None, _P(alpha.ctypes.data),
        _P(beta.ctypes.data), _P(cap.ctypes.data), alpha.size, C, _P(tasks.ctypes.data), n,
        _P(core_begin.ctypes.data), _P(load.ctypes.data)))
    return tasks[:n], core_begin, load


def tasks_to_device(tasks, device) -> torch.Tensor:
    """A TASK_DTYPE array as raw bytes on the device (the ep_task layout)."""
    raw = _np.ascontiguousarray(tasks).view(_np.uint8)
    return torch.from_numpy(raw.copy()).to(device)


def ep_window_copy(src: torch.Tensor, dst: torch.Tensor, row_bytes: int, S: int, C: int,
                   tasks: torch.Tensor | None = None, core_begin: torch.Tensor | None = None,
                   slice_start: torch.Tensor | None = None, core_clock: torch.Tensor | None = None,
                   bad: torch.Tensor | None = None, stream=None) -> None:
    """C persistent cores copy src -> dst rows following task lists (tasks as
    raw ep_task bytes + core_begin i64 [C+1]) or slices (slice_start i64 [C+1])."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.numel() * t.element_size() < S * row_bytes:
            raise ValueError(f"{name} holds fewer than S rows")
    if tasks is not None:
        _need(tasks, "tasks", torch.uint8)
        _need(core_begin, "core_begin", torch.int64, (C + 1,))
    if slice_start is not None:
        _need(slice_start, "slice_start", torch.int64, (C + 1,))
    if core_clock is not None:
        _need(core_clock, "core_clock", torch.int64, (2 * C,))
    if bad is not None:
        _need(bad, "bad", torch.int32, (1,))
    _check(_lib.ep_window_copy(_ptr(src), _ptr(dst), row_bytes, S, _ptr(tasks), _ptr(core_begin),
                               _ptr(slice_start), C, _ptr(core_clock), _ptr(bad),
                               _P(_stream(stream, src.device))))


# ------------------------------------------------------------------- bound calls
class BoundCall:
    """One entry point with its arguments validated and marshalled once.
    Calling it repeats the C call only -- for tight loops, where re-checking
    every tensor would cost more host time than the kernels take.  The
    tensors it refers to are kept alive by the object."""

    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, tuple(args), keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != EP_OK:
            _check(rc)


def bind_route_topk(logits, k, normalize, topk_idx, topk_w, stream) -> BoundCall:
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    _need(topk_idx, "topk_idx", torch.int32, (T, k))
    _need(topk_w, "topk_w", torch.float32, (T, k))
    return BoundCall(_lib.ep_route_topk,
                     (_ptr(logits), T, E, k, int(bool(normalize)), _ptr(topk_idx),
                      _ptr(topk_w), _P(_stream(stream, logits.device))),
                     (logits, topk_idx, topk_w, stream))


def bind_dispatch_layout(topk_idx, E, R, out, stream) -> BoundCall:
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    ws = out["workspace"]
    _need(ws, "workspace", torch.uint8)
    for name, shape in (("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                        ("rank_counts", (R,)), ("rank_offsets", (R + 1,)), ("pos", (T, k))):
        _need(out[name], name, torch.int32, shape)
    if out.get("slot_src") is not None:
        _need(out["slot_src"], "slot_src", torch.int32, (T * k,))
    return BoundCall(_lib.ep_dispatch_layout,
                     (_ptr(topk_idx), T, k, E, R, _ptr(out["expert_counts"]),
                      _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
                      _ptr(out["rank_offsets"]), _ptr(out["pos"]), _ptr(out.get("slot_src")),
                      _ptr(ws), ws.numel(), _P(_stream(stream, topk_idx.device))),
                     (topk_idx, out, stream))


def bind_dispatch(x, pos, send, stream) -> BoundCall:
    _bits_ok(x, "x")
    T, H = x.shape
    _need(pos, "pos", torch.int32)
    k = pos.shape[1]
    if pos.shape[0] != T:
        raise ValueError("pos must be [T][k]")
    _bits_ok(send, "send", (T * k, H))
    return BoundCall(_lib.ep_dispatch,
                     (_ptr(x), T, H, k, _ptr(pos), _ptr(send), _P(_stream(stream, x.device))),
                     (x, pos, send, stream))


def bind_combine(y, pos, topk_w, out, stream) -> BoundCall:
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(y, "y")
    H = y.shape[1]
    if y.shape[0] != T * k:
        raise ValueError("y must have T*k rows")
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _bits_ok(out, "out", (T, H))
    return BoundCall(_lib.ep_combine,
                     (_ptr(y), _ptr(pos), _ptr(topk_w), T, H, k, _ptr(out),
                      _P(_stream(stream, y.device))),
                     (y, pos, topk_w, out, stream))


def bind_combine_grad(grad_out, y, pos, topk_w, grad_y, grad_w, stream) -> BoundCall:
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(grad_out, "grad_out")
    H = grad_out.shape[1]
    if grad_out.shape[0] != T:
        raise ValueError("grad_out must be [T][H]")
    _bits_ok(y, "y", (T * k, H))
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _bits_ok(grad_y, "grad_y", (T * k, H))
    _need(grad_w, "grad_w", torch.float32, (T, k))
    return BoundCall(_lib.ep_combine_grad,
                     (_ptr(grad_out), _ptr(y), _ptr(pos), _ptr(topk_w), T, H, k, _ptr(grad_y),
                      _ptr(grad_w), _P(_stream(stream, y.device))),
                     (grad_out, y, pos, topk_w, grad_y, grad_w, stream))


def bind_dispatch_grad(grad_send, pos, grad_x, stream) -> BoundCall:
    _need(pos, "pos", torch.int32)
    T, k = pos.shape
    _bits_ok(grad_send, "grad_send")
    H = grad_send.shape[1]
    if grad_send.shape[0] != T * k:
        raise ValueError("grad_send must have T*k rows")
    _bits_ok(grad_x, "grad_x", (T, H))
    return BoundCall(_lib.ep_dispatch_grad,
                     (_ptr(grad_send), _ptr(pos), T, H, k, _ptr(grad_x),
                      _P(_stream(stream, grad_send.device))),
                     (grad_send, pos, grad_x, stream))


def ep_set_timing_events(start_event, stop_event) -> None:
    """Bracket the next entry point's kernels with two hipEvent_t handles
    (raw pointers; see HipEvents) -- the kernels' own start and end times."""
    _check(_lib.ep_set_timing_events(_P(start_event), _P(stop_event)))


class HipEvents:
    """Minimal hipEvent_t helper over the HIP runtime already loaded in the
    process (created on the current device, with timing)."""

    def __init__(self):
        self._rt = ctypes.CDLL("libamdhip64.so.7")
        self._rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        self._rt.hipEventDestroy.argtypes = [_P]
        self._rt.hipEventSynchronize.argtypes = [_P]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self._rt.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, start: int, stop: int) -> float:
        ms = ctypes.c_float()
        rc = self._rt.hipEventElapsedTime(ctypes.byref(ms), _P(start), _P(stop))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def synchronize(self, ev: int) -> None:
        self._rt.hipEventSynchronize(_P(ev))

    def destroy(self, ev: int) -> None:
        self._rt.hipEventDestroy(_P(ev))


def ep_get_device_error(workspace: torch.Tensor, stream=None) -> int:
    """EP_OK, EP_ERR_DEVICE or EP_ERR_TIMEOUT for the last call on `workspace`."""
    _need(workspace, "workspace", torch.uint8)
    rc = _lib.ep_get_device_error(_ptr(workspace), _P(_stream(stream, workspace.device)))
    if rc in (EP_OK, EP_ERR_DEVICE, EP_ERR_TIMEOUT):
        return rc
    _check(rc)
    return rc
