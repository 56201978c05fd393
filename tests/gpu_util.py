"""Helpers shared by the GPU parity tests: host<->device transfers of bf16 bit
patterns, the oracle reference chain, and the tolerances (derived below)."""
import numpy as np
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    """Name the case before a GPU step (so a fault can be attributed)."""
    print(f"[gpu-test] {msg}", flush=True)


def to_dev_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV).view(
        torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def poison_bits(shape) -> torch.Tensor:
    """A bf16 tensor filled with 0xFFFF (a NaN pattern no input holds)."""
    return torch.full(shape, -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)


# ----------------------------------------------------------------- tolerances
# Route weights.  The kernel evaluates exp(l_j - m) in f32 (HIP expf, a few
# ulp), sums k terms (or E for normalize=0) in f32 and divides once; the
# oracle is exact to one f32 rounding.  Relative error bound:
#   (|l_j - m| + 4 + n_terms) * 2^-24, n_terms = k (normalize=1) or E (=0).
def route_weight_rtol(logits_row_gap: np.ndarray, n_terms: int) -> np.ndarray:
    return (np.abs(logits_row_gap) + 4.0 + n_terms) * 2.0 ** -24


def check_route_weights(w_gpu, w_ref, logits, idx, normalize, E):
    gap = np.take_along_axis(logits, idx, 1).astype(np.float64) - \
        logits[np.arange(len(idx)), idx[:, 0]][:, None].astype(np.float64)
    rtol = route_weight_rtol(gap, idx.shape[1] if normalize else E)
    err = np.abs(w_gpu.astype(np.float64) - w_ref.astype(np.float64))
    bad = err > rtol * np.abs(w_ref.astype(np.float64)) + 1e-30
    assert not bad.any(), (f"{bad.sum()} route weights outside the derived bound; "
                           f"worst rel err {np.max(err / np.abs(w_ref)):.3g}")


# Combine.  The kernel accumulates in f32: a product, then k-1 fused
# multiply-adds, i.e. k roundings, so |acc32 - S| <= g_k * sum_j |w_j y_j| with
# g_k = k u / (1 - k u), u = 2^-24 (recursive-summation bound).  Both results
# are then rounded to bf16 (half an ulp each), so
#   |gpu - ref| <= ulp_bf16(max(|gpu|, |ref|)) + g_k * sum_j |w_j y_j|.
# Where g_k * sum|w y| stays below a quarter ulp (no cancellation), this is
# the 1-ulp contract: max relative error 2^-7 = 7.8e-3 < 8e-3.
def bf16_ulp(a: np.ndarray) -> np.ndarray:
    a = np.abs(a)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def check_combine(out_gpu_bits, ref_bits, y_bits, pos, w, chunk=256):
    T, k = pos.shape
    gam = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    g = wl.bf16_bits_to_f32(out_gpu_bits).astype(np.float64)
    r = wl.bf16_bits_to_f32(ref_bits).astype(np.float64)
    n_exact = 0
    worst = 0.0
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Y = wl.bf16_bits_to_f32(y_bits[pos[t0:t1].reshape(-1)]).astype(np.float64)
        Y = Y.reshape(t1 - t0, k, -1)
        mag = np.einsum("tk,tkh->th", np.abs(w[t0:t1].astype(np.float64)), np.abs(Y))
        gg, rr = g[t0:t1], r[t0:t1]
        ulp = bf16_ulp(np.maximum(np.abs(gg), np.abs(rr)))
        err = np.abs(gg - rr)
        bad = err > ulp + gam * mag
        assert not bad.any(), f"{bad.sum()} combine outputs outside the derived bound"
        clean = gam * mag <= 0.25 * bf16_ulp(rr)
        within_one = err[clean] <= bf16_ulp(rr[clean]) * 1.0000001
        assert within_one.all(), "1-ulp contract broken where no cancellation occurs"
        big = clean & (np.abs(rr) > 0)
        if big.any():
            worst = max(worst, float(np.max(err[big] / np.abs(rr[big]))))
        n_exact += int(np.sum(out_gpu_bits[t0:t1] == ref_bits[t0:t1]))
    assert worst <= 8e-3, worst
    return n_exact / out_gpu_bits.size


# Weight gradient of the backward combine.  grad_w[t][j] is a dot product of
# two bf16 rows over H: every product is exact in f32, so the error is that of
# the f32 additions.  The kernel adds 8 products per 16-byte vector into a
# per-lane sum over the lane's vectors (at most 8 * ceil(H / 2048) + 8 terms
# for 4 waves of 64 lanes), then 6 butterfly steps and 3 cross-wave adds; any
# summation tree of depth n has |err| <= g_n * sum_h |g_h y_h| with
# g_n = n u / (1 - n u).  n = ceil(H / 64) + 24 bounds that depth for every H,
# and the oracle's own double sum adds at most H * 2^-53 * sum|g y|.
def check_grad_w(gw_gpu, gw_ref, g_bits, y_bits, pos, chunk=256):
    T, k = pos.shape
    H = g_bits.shape[1]
    n = -(-H // 64) + 24
    gam = n * 2.0 ** -24 / (1 - n * 2.0 ** -24) + H * 2.0 ** -53
    worst = 0.0
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        G = np.abs(wl.bf16_bits_to_f32(g_bits[t0:t1]).astype(np.float64))
        Y = np.abs(wl.bf16_bits_to_f32(y_bits[pos[t0:t1].reshape(-1)]).astype(np.float64))
        mag = np.einsum("th,tkh->tk", G, Y.reshape(t1 - t0, k, H))
        err = np.abs(gw_gpu[t0:t1].astype(np.float64) - gw_ref[t0:t1])
        bad = err > gam * mag
        assert not bad.any(), (f"{bad.sum()} weight gradients outside the derived bound; "
                               f"worst {np.max(err / np.maximum(mag, 1e-300)):.3g} x sum|g y|")
        worst = max(worst, float(np.max(err / np.maximum(mag, 1e-300))))
    return worst


# ----------------------------------------------------------------- oracle chain
class Case:
    """Inputs of one workload plus the oracle's route / layout / dispatch."""

    def __init__(self, w: wl.Workload):
        self.w = w
        inp = wl.make_inputs(w)
        self.logits = inp["logits"]
        self.x = inp["x"]
        self.idx, self.wt = oracle.route_topk(self.logits, w.k, 1)
        self.lay = oracle.dispatch_layout(self.idx, w.E, w.R)
        self._send = None

    @property
    def send(self):
        if self._send is None:
            self._send = oracle.dispatch(self.x, self.lay["pos"])
        return self._send
