"""The seeded input generators: determinism and the stated load shapes."""
import numpy as np

import oracle
from combine_ep_route_topk_amd import workloads as wl


def test_same_seed_same_bytes():
    w = wl.WORKLOADS["tiny"]
    a, b = wl.make_inputs(w), wl.make_inputs(w)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["x"], b["x"])
    assert a["x"].dtype == np.uint16 and a["x"].shape == (w.T, w.H)


def test_zipf_bias_is_a_zipf_law():
    w = wl.WORKLOADS["glm45air"]
    b = wl.expert_bias(w, np.random.default_rng(w.seed)).astype(np.float64)
    p = np.exp(b) / np.exp(b).sum()
    ranks = np.argsort(np.argsort(-p)) + 1
    ref = ranks.astype(np.float64) ** -1.2
    np.testing.assert_allclose(p, ref / ref.sum(), rtol=1e-5)


def test_incast_bias_gives_half_of_assignments_to_hot_experts():
    w = wl.WORKLOADS["incast"]
    idx, _ = oracle.route_topk(wl.make_logits(w), w.k, 1)
    share = np.mean(idx < wl.INCAST_HOT_EXPERTS)
    assert 0.495 <= share <= 0.505, share
    assert wl.INCAST_HOT_EXPERTS == round(0.1 * w.E)


def test_bf16_input_rounding_is_nearest_even():
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3.4e38, np.inf], np.float32)
    assert wl.f32_to_bf16_bits(f).tolist() == [0x3F80, 0x3F82, 0x8000, 0x7F80, 0x7F80]
