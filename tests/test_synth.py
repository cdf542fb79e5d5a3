"""The seeded generators produce the shapes and routing structure of the workloads."""

import numpy as np

from synth import WORKLOADS, Workload, make_inputs, make_routing


def test_routing_shapes_distinct_and_gates_normalised():
    for name in ("tiny_f32", "prefill_bf16", "decode_bf16", "fwdbwd_bf16"):
        w = WORKLOADS[name]
        ids, g, _ = make_routing(w)
        assert ids.shape == (w.T, w.K) and ids.dtype == np.int32
        assert g.shape == (w.T, w.K) and g.dtype == np.float32
        assert ((ids >= 0) & (ids < w.E)).all()
        assert all(len(set(r)) == w.K for r in ids[:512])
        np.testing.assert_allclose(g.sum(1), 1.0, rtol=1e-6)


def test_skewed_routing_is_zipf_with_empties_and_ragged_tiles():
    w = WORKLOADS["skewed_bf16"]
    ids, g, _ = make_routing(w)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert (counts == 0).sum() == w.n_empty
    live = np.sort(counts[counts > 0])[::-1]
    assert live[0] > 3 * counts.mean()  # a hot expert
    assert live[0] <= w.T  # distinct ids: at most one slot per token
    assert any(c % 128 for c in live)  # per-expert tails for any tile height


def test_prefill_counts_match_uniform_expectation():
    w = WORKLOADS["prefill_bf16"]
    ids, _, _ = make_routing(w)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert counts.sum() == w.T * w.K
    assert 300 < counts.min() and counts.max() < 470


def test_inputs_are_deterministic_and_prefix_stable():
    w = Workload("d", 101, T=50, H=32, I=16, E=4, K=2)
    a = make_inputs(w)
    b = make_inputs(w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # fewer tokens: x rows are a prefix of the longer draw
    c = make_inputs(w.with_(T=20))
    np.testing.assert_array_equal(c["x"], a["x"][:20])


def test_weight_scale_is_one_over_sqrt_fan_in():
    w = Workload("s", 102, T=4, H=256, I=128, E=2, K=1, dtype="f32")
    inp = make_inputs(w)
    assert abs(inp["up_proj"].std() - 1 / np.sqrt(256)) < 0.003
    assert abs(inp["down_proj"].std() - 1 / np.sqrt(128)) < 0.003
