"""Find the hot-expert logit bias of the skewed-incast workload.

The workload asks for 10% of the 256 experts (experts 0..25) to receive 50% of
all top-8 assignments.  This script bisects the bias added to those experts'
logits, routing with the CPU oracle only, at the workload's fixed seed, and
prints the value stored as workloads.INCAST_HOT_BIAS.

    python tests/golden/calibrate_incast_bias.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))

import oracle  # noqa: E402
from combine_ep_route_topk_amd import workloads as wl  # noqa: E402


def hot_share(bias: float) -> float:
    w = wl.WORKLOADS["incast"]
    logits = wl.make_logits(w, incast_bias=bias)
    idx, _ = oracle.route_topk(logits, w.k, normalize=1)
    return float(np.mean(idx < wl.INCAST_HOT_EXPERTS))


def main():
    lo, hi = 0.0, 4.0
    for _ in range(16):
        mid = (lo + hi) / 2
        s = hot_share(mid)
        print(f"bias={mid!r} hot_share={s:.5f}", flush=True)
        if s < 0.5:
            lo = mid
        else:
            hi = mid
    print(f"INCAST_HOT_BIAS = {mid!r}  (hot share {hot_share(mid):.5f})")


if __name__ == "__main__":
    main()
