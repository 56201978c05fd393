"""Helpers shared by the GPU parity tests: host<->device transfers of bf16 bit
patterns, the oracle reference chain, the bit-equality check of combine-type
outputs, and the tolerances that remain (route weights and the weight
gradient, derived below)."""
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


# Combine.  The contract is the oracle's fp32 chain (HyperParallel-MoE sec.
# 4.1, read as fp32 accumulation in the fixed top-k order): acc = w0*y0 in
# fp32, then fmaf(wj, yj, acc) for j = 1..k-1, then one RNE to bf16.  Every
# GPU path computes exactly that, so the bar is bit equality.  A NaN output
# compares as NaN: which quiet-NaN pattern an operation yields is left open
# by IEEE 754 and is not part of the contract.
def nan_bits(b: np.ndarray) -> np.ndarray:
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def assert_same_bits(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = (got != ref) & ~(nan_bits(got) & nan_bits(ref))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs differ from the "
                             f"oracle's fp32 chain; first at {i}: got {int(got[i]):#06x}, "
                             f"oracle {int(ref[i]):#06x}")


def _ordered(b: np.ndarray) -> np.ndarray:
    """bf16 patterns -> integers in the order of their values (+-0 -> 0), so a
    difference of two is their distance in ulps."""
    mag = (b & 0x7FFF).astype(np.int64)
    return np.where(b & 0x8000, -mag, mag)


def accuracy_vs_exact(got: np.ndarray, exact: np.ndarray, what: str) -> dict:
    """Informational, not a bar: how far the fp32 chain lands from one
    rounding of the exact sum.  Reports the bit-identical fraction, how many
    outputs are more than 1 bf16 ulp away, and the largest distance."""
    ok = ~(nan_bits(got) | nan_bits(exact))
    d = np.abs(_ordered(got[ok]) - _ordered(exact[ok]))
    rep = dict(identical=float(np.mean(d == 0)) if d.size else 1.0,
               over_1ulp=int(np.sum(d > 1)), max_ulp=int(d.max()) if d.size else 0)
    say(f"{what}: {rep['identical']:.6f} of outputs identical to the exact sum; "
        f"{rep['over_1ulp']} more than 1 ulp away (largest {rep['max_ulp']} ulp)")
    return rep


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
