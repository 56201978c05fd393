"""The step captured in a HIP graph (torch.cuda.CUDAGraph over the library's
entry points on a side stream) and replayed: every replay gives the oracle's
results, also when the program's own eager work changes the captured input
buffers and runs other library calls between the replays.

The library launches only kernels -- no memory set or copy nodes -- so a
replay re-runs exactly the eager step's kernels, including the layout's
in-kernel reset of its workspace state."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_route_topk_amd import workloads as wl

from gpu_util import DEV, bits, say, to_dev_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def epm():
    from combine_ep_route_topk_amd import ep as mod
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return mod


@pytest.mark.parametrize("name", ["tiny", "decode", "glm45air", "dsv3"])
def test_graph_replays_match_oracle(epm, name):
    w = wl.WORKLOADS[name]
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    s = torch.cuda.Stream()
    logits = torch.from_numpy(wl.make_logits(w)).to(DEV)
    x = to_dev_bits(wl.make_rows(T, H, w.seed))
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, k), dtype=torch.float32, device=DEV)
    lay = epm.layout_outputs(T, k, E, R, DEV, slot_src=True)
    send = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ops = [epm.bind_route_topk(logits, k, True, idx, wt, s),
           epm.bind_dispatch_layout(idx, E, R, lay, s),
           epm.bind_dispatch(x, lay["pos"], send, s),
           epm.bind_combine(send, lay["pos"], wt, out, s)]
    s.wait_stream(torch.cuda.current_stream())
    for op in ops:
        op()
    s.synchronize()
    say(f"graph capture {w.describe()}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for op in ops:
            op()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: new logits and rows in the captured
        # buffers, and an unrelated eager chain on other buffers
        rng = np.random.default_rng(1000 + rep)
        new_logits = rng.standard_normal((T, E), dtype=np.float32)
        new_x = wl.make_rows(T, H, 2000 + rep)
        logits.copy_(torch.from_numpy(new_logits).to(DEV))
        x.copy_(to_dev_bits(new_x))
        i2, w2 = epm.ep_route_topk(logits, k)
        l2 = epm.ep_dispatch_layout(i2, E, R)
        torch.cuda.synchronize()
        say(f"graph replay {rep} {name}")
        g.replay()
        torch.cuda.synchronize()
        o_idx, o_w = oracle.route_topk(new_logits, k, 1)
        o_lay = oracle.dispatch_layout(o_idx, E, R)
        np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
        for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos",
                    "slot_src"):
            np.testing.assert_array_equal(lay[key].cpu().numpy(), o_lay[key], err_msg=key)
        assert epm.ep_get_device_error(lay["workspace"]) == epm.EP_OK
        assert np.array_equal(bits(out), new_x), f"replay {rep}: combine(dispatch(x)) != x"
        # the eager chain on its own buffers agrees with the replay
        np.testing.assert_array_equal(l2["pos"].cpu().numpy(), o_lay["pos"])
    del g
