"""GPU parity of the backward pass against the CPU oracle.

HyperParallel-MoE sec. 2.2, Fig. 2(b): the backward Dispatch is the gradient
of the forward Combine (ep_combine_grad: grad_y and grad_w), the backward
Combine returns the input activations' gradient (ep_dispatch_grad).

Bars: grad_y bit-exact (the exact product rounded once, also where the f32
product sits on a bf16 tie -- planted in every other token); grad_w within the
derived dot-product bound (gpu_util.check_grad_w) and the same bits on a second
call; grad_x bit-exact against the oracle's fp32 sum in pick order (the
combine chain with unit weights).  Full workload sizes use the launch
configuration the benchmark times; the skewed incast workload is checked on a
sample of tokens, the tokens with the most picks of hot experts among them.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl
from exact_bf16 import plant_tie_products

from gpu_util import (DEV, accuracy_vs_exact, assert_same_bits, bits, check_grad_w, poison_bits,
                      say, to_dev_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


def backward_inputs(T, H, E, R, k, seed, logits=None):
    """pos and weights from the oracle's route + layout; grad_out, expert
    outputs and send-buffer gradients ~ N(0, 1) in bf16; f32-tie products
    planted at pick 0, column 0 of every other token."""
    rng = np.random.default_rng(seed)
    if logits is None:
        logits = rng.standard_normal((T, E), dtype=np.float32)
    idx, w = oracle.route_topk(logits, k, 1)
    pos = oracle.dispatch_layout(idx, E, R)["pos"]
    g = wl.make_rows(T, H, seed + 1)
    plant_tie_products(w, g, range(0, T, 2), seed + 2)
    y = wl.make_rows(T * k, H, seed + 3)
    return pos, w, g, y


def sub_problem(pos, w, g, y, tokens):
    """The listed tokens as a problem of their own: their picks' rows of y,
    in pick order, with pos = 0..n*k-1.  Every gradient the oracle forms is
    per pick (grad_y, grad_w) or per token (grad_x), so the sub-problem's
    gradients are the full problem's at those tokens."""
    k = pos.shape[1]
    rows = pos[tokens].reshape(-1)
    return (np.arange(len(tokens) * k, dtype=np.int32).reshape(-1, k), w[tokens], g[tokens],
            y[rows], rows)


def run_and_check(epm, pos, w, g, y, label, sample=None):
    """sample: check only these tokens against the oracle (all when None)."""
    T, k = pos.shape
    H = g.shape[1]
    say(f"combine_grad {label}")
    d_pos = torch.from_numpy(pos).to(DEV)
    d_w = torch.from_numpy(w).to(DEV)
    d_g, d_y = to_dev_bits(g), to_dev_bits(y)
    gy = poison_bits((T * k, H))
    gw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    epm.ep_combine_grad(d_g, d_y, d_pos, d_w, grad_y=gy, grad_w=gw)
    torch.cuda.synchronize()
    gw1 = gw.cpu().numpy().copy()
    if sample is None:
        r_pos, r_w, r_g, r_y, rows, toks = pos, w, g, y, slice(None), slice(None)
    else:
        r_pos, r_w, r_g, r_y, rows = sub_problem(pos, w, g, y, sample)
        toks = sample
    r_gy, r_gw = oracle.combine_grad(r_g, r_y, r_pos, r_w)
    # with a sample, row i*k+j of the sub-problem's grad_y is pick j of sampled
    # token i, which the full problem holds at row pos[t][j] (= rows[i*k+j])
    assert np.array_equal(bits(gy)[rows], r_gy), "grad_y differs from the exact product"
    check_grad_w(gw1[toks], r_gw, r_g, r_y, r_pos)
    # a second call: the same bits (fixed summation order)
    epm.ep_combine_grad(d_g, d_y, d_pos, d_w, grad_y=gy, grad_w=gw)
    torch.cuda.synchronize()
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), gw1.view(np.uint32))
    del gy, r_gy

    say(f"dispatch_grad {label}")
    gx = poison_bits((T, H))
    epm.ep_dispatch_grad(d_y, d_pos, grad_x=gx)
    torch.cuda.synchronize()
    got = bits(gx)[toks]
    assert_same_bits(got, oracle.dispatch_grad(r_y, r_pos), f"dispatch_grad {label}")
    accuracy_vs_exact(got, oracle.dispatch_grad_exact(r_y, r_pos), f"dispatch_grad {label}")


@pytest.mark.parametrize("name", ["tiny", "decode", "glm45air", "dsv3"])
def test_backward_workloads(epm, name):
    wk = wl.WORKLOADS[name]
    pos, w, g, y = backward_inputs(wk.T, wk.H, wk.E, wk.R, wk.k, wk.seed + 7,
                                   logits=wl.make_logits(wk))
    run_and_check(epm, pos, w, g, y, wk.describe())


def test_backward_incast_sampled(epm):
    """The skewed incast workload (10% of the experts take half of the picks)
    with random expert outputs and signed weights, at full size on the GPU;
    10,240 tokens checked against the oracle: the 5,120 with the most picks of
    hot experts and 5,120 drawn at random from the rest."""
    wk = wl.WORKLOADS["incast"]
    logits = wl.make_logits(wk)
    pos, w, g, y = backward_inputs(wk.T, wk.H, wk.E, wk.R, wk.k, wk.seed + 7, logits=logits)
    w = w - np.float32(0.3)                # signed weights
    idx, _ = oracle.route_topk(logits, wk.k, 1)
    hot = np.sum(idx < wl.INCAST_HOT_EXPERTS, axis=1)
    by_hot = np.argsort(-hot, kind="stable")
    rest = np.random.default_rng(wk.seed + 9).permutation(by_hot[5120:])[:5120]
    sample = np.sort(np.concatenate([by_hot[:5120], rest])).astype(np.int64)
    assert hot[by_hot[:5120]].min() >= 4
    run_and_check(epm, pos, w, g, y, wk.describe() + " (10,240 sampled tokens)", sample=sample)


BACKWARD_EDGE = [
    # T, H, E, R, k, seed
    (1, 8, 1, 1, 1, 301),           # one token, one vector per row
    (3, 16, 4, 2, 2, 302),
    (130, 7176, 64, 8, 6, 303),     # ragged last segment, k = 6 path
    (500, 2048, 32, 8, 4, 308),     # k = 4 path
    (200, 1032, 32, 4, 5, 309),     # runtime-k path, ragged last segment
    (257, 520, 16, 4, 8, 304),      # k = 8 path, ragged segment, odd token count
    (64, 4096, 64, 64, 64, 305),    # the largest k
    (1000, 64, 256, 32, 8, 306),    # short rows, many tokens
    (3, 1 << 20, 4, 2, 2, 307),     # H = 2^20 (maximum): 2 MiB rows
]


@pytest.mark.parametrize("T,H,E,R,k,seed", BACKWARD_EDGE)
def test_backward_edge_shapes(epm, T, H, E, R, k, seed):
    pos, w, g, y = backward_inputs(T, H, E, R, k, seed)
    run_and_check(epm, pos, w, g, y, f"T={T} H={H} E={E} R={R} k={k} seed={seed}")


@pytest.mark.parametrize("k", [4, 5])
def test_backward_grad_w_outside_the_buffer_is_zero_with_infinite_grad(epm, k):
    """grad_w of a pick outside [0, T*k) is exactly 0 even when grad_out
    holds an infinity (0 times infinity would be NaN), on the compile-time
    (k = 4) and runtime (k = 5) pick paths; the other picks' grad_w equal a
    dot product with no invalid row in it, so they do not depend on the
    invalid picks."""
    T, H, E, R = 40, 1024, 16, 4
    pos, w, g, y = backward_inputs(T, H, E, R, k, 321 + k)
    g = g.copy()
    g[:, 5] = 0x7F80                      # +inf (bf16) in every token's row
    pos_bad = pos.copy()
    bad = [(2, 0), (9, k - 1), (30, 2)]
    for t, j in bad:
        pos_bad[t, j] = -1
    say(f"backward, invalid pos with an infinite grad_out, T={T} H={H} k={k}")
    gw = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    gy = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    epm.ep_combine_grad(to_dev_bits(g), to_dev_bits(y), torch.from_numpy(pos_bad).to(DEV),
                        torch.from_numpy(w).to(DEV), grad_y=gy, grad_w=gw)
    torch.cuda.synchronize()
    gw_np = gw.cpu().numpy()
    for t, j in bad:
        assert gw_np[t, j] == 0.0 and not np.signbit(gw_np[t, j])
    _, r_gw = oracle.combine_grad(g, y, pos, w)
    mask = np.ones((T, k), bool)
    for t, j in bad:
        mask[t, j] = False
    np.testing.assert_array_equal(np.isnan(gw_np[mask]), np.isnan(r_gw[mask]))
    np.testing.assert_array_equal(np.isinf(gw_np[mask]), np.isinf(r_gw[mask]))


def test_backward_skips_rows_outside_the_buffer(epm):
    """A pos entry outside [0, T*k): grad_w = 0, no grad_y row written, and no
    contribution to grad_x."""
    T, H, E, R, k = 48, 1024, 16, 4, 4
    pos, w, g, y = backward_inputs(T, H, E, R, k, 311)
    say(f"backward with invalid pos T={T} H={H} k={k}")
    bad = [(3, 1), (17, 0), (40, 3)]
    pos_bad = pos.copy()
    lost = []
    for t, j in bad:
        lost.append(pos[t, j])
        pos_bad[t, j] = -1 if t != 17 else T * k + 5
    d_pos = torch.from_numpy(pos_bad).to(DEV)
    gy = poison_bits((T * k, H))
    gw = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    epm.ep_combine_grad(to_dev_bits(g), to_dev_bits(y), d_pos, torch.from_numpy(w).to(DEV),
                        grad_y=gy, grad_w=gw)
    gx = poison_bits((T, H))
    epm.ep_dispatch_grad(to_dev_bits(y), d_pos, grad_x=gx)
    torch.cuda.synchronize()
    r_gy, r_gw = oracle.combine_grad(g, y, pos, w)
    got = bits(gy)
    keep = np.setdiff1d(np.arange(T * k), lost)
    assert np.array_equal(got[keep], r_gy[keep])
    assert np.all(got[lost] == 0xFFFF), "a row outside the buffer's picks was written"
    gw_np = gw.cpu().numpy()
    for t, j in bad:
        assert gw_np[t, j] == 0.0
    mask = np.ones((T, k), bool)
    for t, j in bad:
        mask[t, j] = False
    check_grad_w(np.where(mask, gw_np, 0.0), np.where(mask, r_gw, 0.0), g, y, pos)
    # expected grad_x: the lost picks' rows count as zero
    y0 = y.copy()
    y0[lost] = 0
    assert_same_bits(bits(gx), oracle.dispatch_grad(y0, pos), "dispatch_grad with picks outside")


@pytest.mark.parametrize("T,H,E,R,k,seed", [(4099, 4096, 64, 8, 8, 321),
                                             (4097, 7168, 64, 8, 6, 322)])
def test_backward_large_skips_rows_outside_the_buffer(epm, T, H, E, R, k, seed):
    """The same at sizes that take the capped, evenly rounded scatter grid
    (more than 64 MiB of grad_y; 8 and 7 vectors per lane), with a last group
    of tokens that is not full: every kept row bit-exact, the lost rows
    untouched, grad_w = 0 for the lost picks and within the bound elsewhere."""
    pos, w, g, y = backward_inputs(T, H, E, R, k, seed)
    picks = [(0, 0, -1), (T // 2, k - 1, T * k), (T - 1, 1, T * k + 3)]
    bad = pos.copy()
    lost = []
    for t, j, v in picks:
        lost.append(pos[t, j])
        bad[t, j] = v
    say(f"combine_grad (capped grid) with invalid pos T={T} H={H} k={k}")
    gy = poison_bits((T * k, H))
    gw = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    epm.ep_combine_grad(to_dev_bits(g), to_dev_bits(y), torch.from_numpy(bad).to(DEV),
                        torch.from_numpy(w).to(DEV), grad_y=gy, grad_w=gw)
    torch.cuda.synchronize()
    r_gy, r_gw = oracle.combine_grad(g, y, pos, w)
    got = bits(gy)
    keep = np.setdiff1d(np.arange(T * k), lost)
    assert np.array_equal(got[keep], r_gy[keep])
    assert np.all(got[lost] == 0xFFFF), "a row outside the buffer's picks was written"
    gw_np = gw.cpu().numpy()
    mask = np.ones((T, k), bool)
    for t, j, _ in picks:
        mask[t, j] = False
        assert gw_np[t, j] == 0.0
    check_grad_w(np.where(mask, gw_np, 0.0), np.where(mask, r_gw, 0.0), g, y, pos)


def test_backward_validation(epm):
    T, H, k = 4, 16, 2
    d = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    w = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        epm.ep_combine_grad(d(T, H), d(T * k + 1, H), pos, w)
    with pytest.raises(ValueError):
        epm.ep_dispatch_grad(d(T * k - 1, H), pos)
    with pytest.raises(epm.EpError):
        epm.ep_dispatch_grad(d(T * k, 12), pos)         # H not a multiple of 8
