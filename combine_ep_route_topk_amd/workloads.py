"""Seeded synthetic workloads for MoE expert-parallel dispatch/combine.

This module only draws inputs: it holds none of the method's arithmetic (no
top-k, no counting, no prefix sums, no reduction), so the CPU oracle and the
HIP library can both be fed from it without sharing any computation.

Shapes follow the pages' workloads:
  * H = 7168, top-8, 256 routed experts -- the DeepSeek-style rows of UBEP's
    Table 3 (evaluated models) and the EP=32, 4096-tokens-per-batch,
    H = 7168, top-8 dispatch/combine microbenchmark of StrataCL's Table 2;
  * H = 4096, 128 experts, top-8 with skewed expert load -- the GLM-4.5-Air
    routing that RailWave replays (sec. "Communication bottlenecks with fixed
    routing"; its traces are not available, a Zipf bias stands in);
  * 16384 tokens with 10% of experts taking half of the assignments -- a
    one-GPU stand-in for the receiver-incast case RailWave describes.

Draw order for every config, from numpy's PCG64 ``default_rng(seed)``:
  1. (GLM-like only) a permutation of the experts that fixes the Zipf ranks;
  2. logits f32 [T][E] ~ N(0, 1), plus the config's per-expert bias;
  3. x f32 [T][H] ~ N(0, 1), rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import numpy as np

# Bias added to the logits of the 26 hot experts (experts 0..25, 10% of 256) of
# the skewed-incast config so that they receive 50% (+-0.5%) of all top-8
# assignments at seed 1005.  Found by bisection with the CPU oracle's router by
# tests/golden/calibrate_incast_bias.py; tests/test_workloads.py re-checks it.
INCAST_HOT_BIAS = 1.10394287109375
INCAST_HOT_EXPERTS = 26


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # hidden size (bf16 elements per row)
    E: int          # experts
    R: int          # virtual EP ranks (E % R == 0)
    k: int          # top-k
    seed: int
    bias: str = "none"      # "none" | "zipf1.2" | "incast"
    fused: bool = False     # the config is run in the flag-in-payload fused mode

    @property
    def S(self) -> int:
        return self.T * self.k

    def describe(self) -> str:
        return (f"{self.name}: T={self.T} H={self.H} E={self.E} R={self.R} "
                f"k={self.k} seed={self.seed} bias={self.bias}")


WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, E=8, R=2, k=2, seed=1001),
    "decode": Workload("decode", T=128, H=7168, E=256, R=32, k=8, seed=1002),
    "glm45air": Workload("glm45air", T=4096, H=4096, E=128, R=16, k=8, seed=1003,
                         bias="zipf1.2"),
    "dsv3": Workload("dsv3", T=4096, H=7168, E=256, R=32, k=8, seed=1004),
    "incast": Workload("incast", T=16384, H=7168, E=256, R=64, k=8, seed=1005,
                       bias="incast", fused=True),
}
ORDER = ["tiny", "decode", "glm45air", "dsv3", "incast"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest, ties to even); returns the uint16 patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def expert_bias(w: Workload, rng: np.random.Generator | None = None,
                incast_bias: float | None = None) -> np.ndarray:
    """Per-expert logit bias (f32 [E]).  Draws the Zipf permutation from rng."""
    E = w.E
    if w.bias == "none":
        return np.zeros(E, np.float32)
    if w.bias == "zipf1.2":
        # b_e = ln p_e with p_e proportional to rank_e^-1.2: softmax(b) is the
        # Zipf(1.2) law over experts; rank_e comes from a seeded permutation.
        perm = rng.permutation(E)
        rank = np.empty(E, np.int64)
        rank[perm] = np.arange(1, E + 1)
        p = rank.astype(np.float64) ** -1.2
        p /= p.sum()
        return np.log(p).astype(np.float32)
    if w.bias == "incast":
        b = np.zeros(E, np.float32)
        b[:INCAST_HOT_EXPERTS] = INCAST_HOT_BIAS if incast_bias is None else incast_bias
        return b
    raise ValueError(w.bias)


def make_logits(w: Workload, incast_bias: float | None = None) -> np.ndarray:
    return make_inputs(w, with_x=False, incast_bias=incast_bias)["logits"]


def make_inputs(w: Workload, with_x: bool = True, incast_bias: float | None = None):
    """Returns dict(logits f32 [T][E], x u16 [T][H] bf16 bits)."""
    rng = np.random.default_rng(w.seed)
    bias = expert_bias(w, rng, incast_bias)
    logits = rng.standard_normal((w.T, w.E), dtype=np.float32)
    logits += bias[None, :]
    out = {"logits": logits}
    if with_x:
        x = rng.standard_normal((w.T, w.H), dtype=np.float32)
        out["x"] = f32_to_bf16_bits(x)
    return out


def make_rows(n: int, H: int, seed: int) -> np.ndarray:
    """n bf16 rows ~ N(0, 1) (e.g. synthetic expert outputs) -> u16 [n][H]."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((n, H), dtype=np.float32))


def random_topk(T: int, E: int, k: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Distinct random experts per token and positive weights (not normalized),
    for kernel tests that do not go through the router."""
    rng = np.random.default_rng(seed)
    keys = rng.random((T, E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = rng.random((T, k), dtype=np.float32) + np.float32(0.01)
    return idx, w


def algorithmic_bytes(w: Workload) -> dict:
    """Bytes the method must move per call, per op (no padding, no staging).

    dispatch: read x (2H per token) + pos (4k), write k rows (2Hk)
    combine : read k rows (2Hk) + pos (4k) + weights (4k), write out (2H)
    route   : read logits (4E), write idx + weights (8k)
    layout  : read idx (4k), write pos + slot_src (8k) per token, plus the
              per-expert / per-rank arrays.
    """
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    return {
        "dispatch": T * (2 * H * (1 + k) + 4 * k),
        "combine": T * (2 * H * (k + 1) + 8 * k),
        "route": T * (4 * E + 8 * k),
        "layout": T * (12 * k) + 4 * (2 * E + 1) + 4 * (2 * R + 1),
    }



def algorithmic_bytes_backward(w: Workload) -> dict:
    """Bytes the backward pass must move per call, per op.

    combine_grad : read grad_out (2H per token) + k rows of y (2Hk) + pos and
                   weights (8k), write k gradient rows (2Hk) + grad_w (4k)
    dispatch_grad: read k rows (2Hk) + pos (4k), write grad_x (2H)
    """
    T, H, k = w.T, w.H, w.k
    return {
        "combine_grad": T * (2 * H * (1 + 2 * k) + 12 * k),
        "dispatch_grad": T * (2 * H * (k + 1) + 4 * k),
    }
