"""CPU oracle for MoE expert-parallel route / dispatch / combine.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg -- never by the product package, which has no CPU
fallback.  The arithmetic lives in ep_oracle.c (plain C, double precision);
this module only marshals numpy arrays into it.  Page citations for each
function are in ep_oracle.h.

parity pins: every function here is pinned by the CPU tests in
tests/test_oracle_*.py against closed forms, brute force, library routines
and hand-derived fixtures under tests/golden/.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libep_oracle.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.ep_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.ep_oracle_bf16_to_double.restype = ctypes.c_double
        L.ep_oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.ep_oracle_double_to_bf16.restype = ctypes.c_uint16
        L.ep_oracle_route_topk.argtypes = [P, i64, i32, i32, i32, P, P]
        L.ep_oracle_dispatch_layout.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, P]
        L.ep_oracle_dispatch.argtypes = [P, i64, i32, i32, P, P]
        L.ep_oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
        L.ep_oracle_combine_exact.argtypes = [P, P, P, i64, i32, i32, P]
        L.ep_oracle_combine_tokens.argtypes = [P, P, P, i64, i32, i32, P, i64, P]
        L.ep_oracle_fused_trailer.argtypes = [ctypes.c_uint64, P, i64, P]
        L.ep_oracle_combine_grad.argtypes = [P, P, P, P, i64, i32, i32, P, P]
        L.ep_oracle_dispatch_grad.argtypes = [P, P, i64, i32, i32, P]
        L.ep_oracle_dispatch_grad_exact.argtypes = [P, P, i64, i32, i32, P]
        L.ep_oracle_slices.argtypes = [P, i32, i32, P, P, P]
        L.ep_oracle_lpt.argtypes = [P, P, i32, P, i32, i32, P, P, P]
        L.ep_oracle_rank_coalesce.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, P]
        L.ep_oracle_rank_coalesce.restype = i64
        L.ep_oracle_exchange_waves.argtypes = [i32, P]
        L.ep_oracle_expand_records.argtypes = [P, i64, i32, P, P, P]
        L.ep_oracle_incast_degree.argtypes = [P, i32]
        L.ep_oracle_incast_degree.restype = i32
        for f in ("ep_oracle_route_topk", "ep_oracle_dispatch_layout",
                  "ep_oracle_dispatch", "ep_oracle_combine", "ep_oracle_combine_exact",
                  "ep_oracle_dispatch_grad_exact",
                  "ep_oracle_combine_tokens", "ep_oracle_fused_trailer",
                  "ep_oracle_combine_grad", "ep_oracle_dispatch_grad", "ep_oracle_slices",
                  "ep_oracle_lpt"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def bf16_to_double(b: int) -> float:
    return lib().ep_oracle_bf16_to_double(int(b))


def double_to_bf16(v: float) -> int:
    return int(lib().ep_oracle_double_to_bf16(float(v)))


def route_topk(logits, k: int, normalize: int = 1):
    """logits f32 [T][E] -> (topk_idx i32 [T][k], topk_w f32 [T][k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib().ep_oracle_route_topk(_p(logits), T, E, k, int(normalize), _p(idx), _p(w)),
           "route_topk")
    return idx, w


def dispatch_layout(topk_idx, E: int, R: int):
    """topk_idx i32 [T][k] -> dict of the layout arrays."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    out = dict(
        expert_counts=np.empty(E, np.int32),
        expert_offsets=np.empty(E + 1, np.int32),
        rank_counts=np.empty(R, np.int32),
        rank_offsets=np.empty(R + 1, np.int32),
        pos=np.empty((T, k), np.int32),
        slot_src=np.empty(T * k, np.int32),
    )
    _check(lib().ep_oracle_dispatch_layout(
        _p(topk_idx), T, k, E, R, _p(out["expert_counts"]), _p(out["expert_offsets"]),
        _p(out["rank_counts"]), _p(out["rank_offsets"]), _p(out["pos"]), _p(out["slot_src"])),
        "dispatch_layout")
    return out


def dispatch(x_bits, pos, out=None):
    """x bf16 bits u16 [T][H], pos i32 [T][k] -> send u16 [T*k][H]."""
    x_bits = _c(x_bits, np.uint16)
    pos = _c(pos, np.int32)
    T, H = x_bits.shape
    k = pos.shape[1]
    send = out if out is not None else np.empty((T * k, H), np.uint16)
    _check(lib().ep_oracle_dispatch(_p(x_bits), T, H, k, _p(pos), _p(send)), "dispatch")
    return send


def _combine(fn, y_bits, pos, topk_w):
    y_bits = _c(y_bits, np.uint16)
    pos = _c(pos, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = pos.shape
    H = y_bits.shape[1]
    out = np.empty((T, H), np.uint16)
    _check(getattr(lib(), fn)(_p(y_bits), _p(pos), _p(topk_w), T, H, k, _p(out)), fn)
    return out


def combine(y_bits, pos, topk_w):
    """The combine contract: fp32 product for pick 0, fmaf for picks 1..k-1 in
    order, one RNE to bf16.  y u16 [T*k][H] (send order), pos i32 [T][k],
    w f32 [T][k] -> out u16 [T][H]."""
    return _combine("ep_oracle_combine", y_bits, pos, topk_w)


def combine_exact(y_bits, pos, topk_w):
    """The accuracy reference: the exact weighted sum (in double, every
    product exact) rounded once to bf16.  Same arguments as combine."""
    return _combine("ep_oracle_combine_exact", y_bits, pos, topk_w)


def combine_tokens(y_bits, pos, topk_w, tokens):
    """combine (the fp32 chain) for the listed tokens only -> u16 [len(tokens)][H]."""
    y_bits = _c(y_bits, np.uint16)
    pos = _c(pos, np.int32)
    topk_w = _c(topk_w, np.float32)
    tokens = _c(tokens, np.int64)
    T, k = pos.shape
    H = y_bits.shape[1]
    out = np.empty((len(tokens), H), np.uint16)
    _check(lib().ep_oracle_combine_tokens(_p(y_bits), _p(pos), _p(topk_w), T, H, k,
                                          _p(tokens), len(tokens), _p(out)),
           "combine_tokens")
    return out


def combine_grad(grad_out_bits, y_bits, pos, topk_w):
    """Backward of combine: grad_out u16 [T][H], y u16 [T*k][H], pos i32
    [T][k], w f32 [T][k] -> (grad_y u16 [T*k][H], grad_w f64 [T][k])."""
    grad_out_bits = _c(grad_out_bits, np.uint16)
    y_bits = _c(y_bits, np.uint16)
    pos = _c(pos, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, k = pos.shape
    H = grad_out_bits.shape[1]
    grad_y = np.zeros((T * k, H), np.uint16)
    grad_w = np.zeros((T, k), np.float64)
    _check(lib().ep_oracle_combine_grad(_p(grad_out_bits), _p(y_bits), _p(pos), _p(topk_w),
                                        T, H, k, _p(grad_y), _p(grad_w)), "combine_grad")
    return grad_y, grad_w


def _dispatch_grad(fn, grad_send_bits, pos):
    grad_send_bits = _c(grad_send_bits, np.uint16)
    pos = _c(pos, np.int32)
    T, k = pos.shape
    H = grad_send_bits.shape[1]
    grad_x = np.empty((T, H), np.uint16)
    _check(getattr(lib(), fn)(_p(grad_send_bits), _p(pos), T, H, k, _p(grad_x)), fn)
    return grad_x


def dispatch_grad(grad_send_bits, pos):
    """Backward of dispatch, fp32 sum in pick order then one RNE:
    grad_send u16 [T*k][H], pos i32 [T][k] -> grad_x u16 [T][H]."""
    return _dispatch_grad("ep_oracle_dispatch_grad", grad_send_bits, pos)


def dispatch_grad_exact(grad_send_bits, pos):
    """The accuracy reference for dispatch_grad: the sum in double, one RNE."""
    return _dispatch_grad("ep_oracle_dispatch_grad_exact", grad_send_bits, pos)


def slices(expert_offsets, P: int):
    """Equal slot slices for P workers -> (start i64 [P+1], expert i32 [P],
    offset i64 [P])."""
    eo = _c(expert_offsets, np.int32)
    E = eo.shape[0] - 1
    start = np.empty(P + 1, np.int64)
    expert = np.empty(P, np.int32)
    offset = np.empty(P, np.int64)
    _check(lib().ep_oracle_slices(_p(eo), E, P, _p(start), _p(expert), _p(offset)), "slices")
    return start, expert, offset


def lpt(cost, peer, cap_of_peer, C: int):
    """LPT list schedule -> (core i32 [U], stripe i32 [U], load f64 [C])."""
    cost = _c(cost, np.float64)
    peer = _c(peer, np.int32)
    cap = _c(cap_of_peer, np.int32)
    U = cost.shape[0]
    core = np.empty(max(U, 1), np.int32)
    stripe = np.empty(max(U, 1), np.int32)
    load = np.empty(C, np.float64)
    _check(lib().ep_oracle_lpt(_p(cost), _p(peer), U, _p(cap), cap.shape[0], C, _p(core),
                               _p(stripe), _p(load)), "lpt")
    return core[:U], stripe[:U], load


def rank_coalesce(topk_idx, E: int, R: int):
    """One send record per (token, destination rank) -> dict with rank_counts
    i32 [R], rank_offsets i32 [R+1], row_of_pick i32 [T][k], send_pos i32
    [T][k], row_src i32 [C], row_experts u64 [C] (C = rank_offsets[R])."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    S = T * k
    out = dict(rank_counts=np.empty(R, np.int32), rank_offsets=np.empty(R + 1, np.int32),
               row_of_pick=np.empty((T, k), np.int32), send_pos=np.empty((T, k), np.int32),
               row_src=np.empty(max(S, 1), np.int32), row_experts=np.empty(max(S, 1), np.uint64))
    C = lib().ep_oracle_rank_coalesce(_p(idx), T, k, E, R, _p(out["rank_counts"]),
                                      _p(out["rank_offsets"]), _p(out["row_of_pick"]),
                                      _p(out["send_pos"]), _p(out["row_src"]),
                                      _p(out["row_experts"]))
    _check(min(C, 0), "rank_coalesce")
    out["row_src"] = out["row_src"][:C]
    out["row_experts"] = out["row_experts"][:C]
    return out


def expand_records(masks, L: int):
    """Receiver-side expansion of coalesced records -> dict(expert_counts i32
    [L], expert_offsets i32 [L+1], pos i32 [C][L] (-1 where a record does not
    feed that expert))."""
    masks = _c(masks, np.uint64)
    C = masks.shape[0]
    out = dict(expert_counts=np.empty(L, np.int32), expert_offsets=np.empty(L + 1, np.int32),
               pos=np.empty((C, L), np.int32))
    _check(lib().ep_oracle_expand_records(_p(masks) if C else ctypes.c_void_p(8), C, L,
                                          _p(out["expert_counts"]), _p(out["expert_offsets"]),
                                          _p(out["pos"]) if C else ctypes.c_void_p(8)),
           "expand_records")
    return out


def exchange_waves(N: int):
    """Cyclic exchange waves -> i32 [N-1][N]: peer[k-1][s] = (s + k) mod N."""
    peer = np.empty((max(N - 1, 0), N), np.int32)
    _check(lib().ep_oracle_exchange_waves(N, _p(peer) if peer.size else ctypes.c_void_p(1)),
           "exchange_waves")
    return peer


def incast_degree(dst) -> int:
    """Largest number of senders of one wave with the same receiver."""
    dst = _c(dst, np.int32)
    d = lib().ep_oracle_incast_degree(_p(dst), dst.shape[0])
    _check(min(d, 0), "incast_degree")
    return int(d)


def fused_trailers(epoch: int, slot_src):
    """Expected 16-byte trailers of every slot -> u8 [S][16]."""
    slot_src = _c(slot_src, np.int32)
    S = slot_src.shape[0]
    tr = np.empty((S, 16), np.uint8)
    L = lib()
    for s in range(S):
        _check(L.ep_oracle_fused_trailer(ctypes.c_uint64(epoch), _p(slot_src), s,
                                         ctypes.c_void_p(tr.ctypes.data + 16 * s)),
               "fused_trailer")
    return tr
