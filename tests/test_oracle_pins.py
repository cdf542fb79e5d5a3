"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle (``oracle/moe_oracle.c``) is checked here against things other than
itself:

* routing: numpy's bincount / cumsum / stable argsort (library routines), the
  hand-worked fixture ``tests/golden/route_hand.txt`` and the combine protocol
  of the overlap explainer page, section 6 (every token's K branches come back
  exactly once);
* forward: a per-token brute force that uses no routing at all and PyTorch's
  own ``silu`` (library), the K=1 / gate=1 reduction to a dense SwiGLU FFN,
  the E=1 closed form, a scalar closed form with sigmoid(ln 3) = 3/4, and
  invariants (empty experts, token permutation, gate linearity);
* backward: PyTorch autograd in float64 (library), central finite differences
  on the oracle's own forward, and the linearity identities
  <dY, y> = Σ g·d_g = <W2, dW2>.

The routed-expert math follows the HyperMegaMoE issue page (sections 2.1, 2.2,
3.1 and 4.1).  Which half of up_proj's 2I outputs is the SwiGLU gate is not
fixed by the pages; the reading here is "first I columns are the gate".
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import Workload, bf16_bits_from_f32, f32_from_bf16_bits, make_inputs, make_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers
def np_route(ids, E):
    """Routing via numpy library routines only."""
    flat = np.asarray(ids).ravel().astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_slot = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slot)
    slot_pos[sorted_slot] = np.arange(len(flat), dtype=np.int32)
    return counts, offsets, sorted_slot, slot_pos


def small(T, H, I, E, K, dtype="f32", routing="uniform", cfg_id=100, **kw):
    return Workload("pin", cfg_id, T=T, H=H, I=I, E=E, K=K, dtype=dtype, routing=routing, **kw)


def as64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = f32_from_bf16_bits(a)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def brute_forward(x, ids, g, W1, W2):
    """y_t = Σ_k g_tk · (silu(x_t W1[e][:, :I]) ⊙ (x_t W1[e][:, I:])) W2[e], token by token."""
    T, H = x.shape
    K = ids.shape[1]
    I = W2.shape[1]
    y = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            h = x[t] @ W1[e]
            y[t] = y[t] + g[t, k] * ((F.silu(h[:I]) * h[I:]) @ W2[e])
    return y


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300) if b.size else 1.0
    return float(np.abs(a - b).max() / den) if a.size else 0.0


def random_ids(rng, T, K, E, distinct=False):
    if distinct:
        return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32).reshape(T, K)
    return rng.integers(0, E, size=(T, K)).astype(np.int32)


# --------------------------------------------------------------------------- routing
ROUTE_CASES = [
    ("uniform", 257, 3, 16),
    ("k1", 100, 1, 7),
    ("t0", 0, 4, 8),
    ("t1", 1, 6, 64),
    ("e1", 33, 2, 1),
    ("big_e", 300, 8, 1024),
]


@pytest.mark.parametrize("name,T,K,E", ROUTE_CASES)
def test_route_matches_numpy(name, T, K, E):
    rng = np.random.default_rng(abs(hash(name)) % 2**32)
    ids = random_ids(rng, T, K, E)
    got = oracle.route(ids, E)
    want = np_route(ids, E)
    for g_, w_ in zip(got, want):
        np.testing.assert_array_equal(g_, w_)


def test_route_all_one_expert_and_empties():
    T, K, E = 65, 3, 9
    ids = np.full((T, K), 4, np.int32)
    counts, offsets, ss, sp = oracle.route(ids, E)
    assert counts.tolist() == [0, 0, 0, 0, T * K, 0, 0, 0, 0]
    assert offsets.tolist() == [0, 0, 0, 0, 0, T * K, T * K, T * K, T * K, T * K]
    np.testing.assert_array_equal(ss, np.arange(T * K))
    np.testing.assert_array_equal(sp, np.arange(T * K))


def test_route_int64_ids_and_duplicates():
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 5, size=(40, 4)).astype(np.int64)
    assert any(len(set(r)) < 4 for r in ids)  # duplicates present
    got = oracle.route(ids, 5)
    want = np_route(ids, 5)
    for g_, w_ in zip(got, want):
        np.testing.assert_array_equal(g_, w_)


def test_route_zipf_with_forced_empties():
    w = small(T=999, H=8, I=8, E=32, K=8, routing="zipf", n_empty=3)
    ids, gates, _ = make_routing(w)
    counts, offsets, ss, sp = oracle.route(ids, w.E)
    assert (counts == 0).sum() >= 3
    for g_, w_ in zip((counts, offsets, ss, sp), np_route(ids, w.E)):
        np.testing.assert_array_equal(g_, w_)


def test_route_hand_worked_fixture():
    vals = {}
    with open(os.path.join(GOLDEN, "route_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *rest = line.split()
                vals[key] = [int(v) for v in rest]
    T, K, E = vals["T"][0], vals["K"][0], vals["E"][0]
    ids = np.array(vals["ids"], np.int32).reshape(T, K)
    counts, offsets, ss, sp = oracle.route(ids, E)
    assert counts.tolist() == vals["counts"]
    assert offsets.tolist() == vals["offsets"]
    assert ss.tolist() == vals["sorted_slot"]
    assert sp.tolist() == vals["slot_pos"]


def test_route_combine_protocol():
    """Each token's K branches return exactly once (done == K), counts sum to T*K,
    and the permutation is a bijection."""
    rng = np.random.default_rng(3)
    T, K, E = 500, 6, 64
    ids = random_ids(rng, T, K, E, distinct=True)
    counts, offsets, ss, sp = oracle.route(ids, E)
    assert counts.sum() == T * K
    done = np.bincount(ss // K, minlength=T)
    assert (done == K).all()
    assert sorted(ss.tolist()) == list(range(T * K))
    np.testing.assert_array_equal(sp[ss], np.arange(T * K))
    # every slot lands inside its expert's segment
    flat = ids.ravel()
    assert ((offsets[flat] <= sp) & (sp < offsets[flat + 1])).all()


@pytest.mark.parametrize("bad", [-1, 5, 1 << 20])
def test_route_rejects_out_of_range_ids(bad):
    ids = np.zeros((4, 2), np.int32)
    ids[2, 1] = bad
    with pytest.raises(oracle.OracleError):
        oracle.route(ids, 5)


# --------------------------------------------------------------------------- forward
FWD_CASES = [
    # T, H, I, E, K, dtype, distinct
    (7, 8, 6, 4, 3, "f32", False),   # duplicates allowed
    (5, 16, 8, 3, 2, "bf16", True),
    (1, 4, 4, 1, 1, "f32", True),
    (9, 12, 10, 6, 4, "f32", True),
]


@pytest.mark.parametrize("T,H,I,E,K,dtype,distinct", FWD_CASES)
def test_forward_matches_per_token_brute_force(T, H, I, E, K, dtype, distinct):
    w = small(T, H, I, E, K, dtype=dtype)
    inp = make_inputs(w)
    rng = np.random.default_rng(T * 1000 + H)
    ids = random_ids(rng, T, K, E, distinct=distinct)
    g = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    yb = brute_forward(as64(inp["x"]), ids, as64(g), as64(inp["up_proj"]), as64(inp["down_proj"]))
    assert rel_err(y, yb.numpy()) < 1e-12


def test_forward_k1_unit_gate_is_dense_swiglu_ffn():
    """K=1 with gate 1: every token gets exactly the dense SwiGLU FFN of its expert,
    computed here with torch.nn.functional.silu and plain matmuls."""
    T, H, I, E = 12, 16, 24, 3
    w = small(T, H, I, E, 1)
    inp = make_inputs(w)
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)
    g = np.ones((T, 1), np.float32)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    x, W1, W2 = as64(inp["x"]), as64(inp["up_proj"]), as64(inp["down_proj"])
    for e in range(E):
        rows = np.where(ids[:, 0] == e)[0]
        xe = x[rows]
        gate = xe @ W1[e][:, :I]
        up = xe @ W1[e][:, I:]
        dense = (F.silu(gate) * up) @ W2[e]
        assert rel_err(y[rows], dense.numpy()) < 1e-12


def test_forward_single_expert_closed_form():
    """E=1: all K slots hit expert 0, so y = (Σ_k g_k) · FFN(x)."""
    T, H, I, K = 6, 8, 8, 4
    w = small(T, H, I, 1, K, routing="replace")
    inp = make_inputs(w)
    g = np.random.default_rng(1).uniform(0, 1, (T, K)).astype(np.float32)
    ids = np.zeros((T, K), np.int32)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    y1 = oracle.forward(inp["x"], np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                        inp["up_proj"], inp["down_proj"])
    np.testing.assert_allclose(y, g.astype(np.float64).sum(1, keepdims=True) * y1, rtol=1e-13,
                               atol=1e-15)


def test_forward_scalar_closed_form():
    """H = I = 1: y = Σ_k g_k · silu(x·a_e) · (x·b_e) · d_e.  With x·a = ln 3 the
    sigmoid is exactly 3/4, so silu = (3/4)·ln 3."""
    ln3 = math.log(3.0)
    x = np.array([[1.0]], np.float32)
    up = np.array([[[ln3, 2.0]], [[0.0, 5.0]]], np.float32)  # expert 1: silu(0) = 0
    down = np.array([[[0.5]], [[7.0]]], np.float32)
    ids = np.array([[0, 1]], np.int32)
    g = np.array([[0.25, 0.75]], np.float32)
    y = oracle.forward(x, ids, g, up, down)
    a = float(np.float32(ln3))  # the fp32 value actually stored
    sig = 1.0 / (1.0 + math.exp(-a))
    want = 0.25 * (a * sig) * 2.0 * 0.5
    assert abs(y[0, 0] - want) < 1e-15
    assert abs(want - 0.25 * 0.75 * ln3) < 1e-7  # sigmoid(ln 3) = 3/4


def test_forward_empty_expert_weights_are_never_read():
    T, H, I, E, K = 20, 8, 8, 5, 2
    w = small(T, H, I, E, K)
    inp = make_inputs(w)
    rng = np.random.default_rng(5)
    ids = rng.choice([0, 1, 3], size=(T, K)).astype(np.int32)  # experts 2 and 4 empty
    g = rng.uniform(0, 1, (T, K)).astype(np.float32)
    y0 = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    up, down = inp["up_proj"].copy(), inp["down_proj"].copy()
    up[[2, 4]] = np.nan
    down[[2, 4]] = 1e30
    y1 = oracle.forward(inp["x"], ids, g, up, down)
    np.testing.assert_array_equal(y0, y1)


def test_forward_token_permutation_equivariance():
    T, H, I, E, K = 30, 8, 12, 6, 3
    w = small(T, H, I, E, K)
    inp = make_inputs(w)
    ids, g, _ = make_routing(w)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    perm = np.random.default_rng(11).permutation(T)
    yp = oracle.forward(inp["x"][perm], ids[perm], g[perm], inp["up_proj"], inp["down_proj"])
    np.testing.assert_array_equal(yp, y[perm])


def test_forward_gate_linearity():
    T, H, I, E, K = 15, 8, 8, 4, 2
    w = small(T, H, I, E, K)
    inp = make_inputs(w)
    rng = np.random.default_rng(2)
    ids = random_ids(rng, T, K, E, distinct=True)
    g1 = (rng.integers(0, 64, (T, K)) / 64.0).astype(np.float32)  # dyadic: g1+g2 exact
    g2 = (rng.integers(0, 64, (T, K)) / 64.0).astype(np.float32)
    f = lambda g: oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    assert rel_err(f(g1 + g2), f(g1) + f(g2)) < 1e-13


def test_forward_intermediates_follow_permutation():
    T, H, I, E, K = 11, 8, 6, 3, 2
    w = small(T, H, I, E, K)
    inp = make_inputs(w)
    ids, g, _ = make_routing(w)
    y, it = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"], intermediates=True)
    x, W1, W2 = as64(inp["x"]), as64(inp["up_proj"]), as64(inp["down_proj"])
    for p in range(T * K):
        s = it["sorted_slot"][p]
        t, e = s // K, ids.ravel()[s]
        h = x[t] @ W1[e]
        act = F.silu(h[:I]) * h[I:]
        assert rel_err(it["act"][p], act.numpy()) < 1e-12
        assert rel_err(it["o"][p], (act @ W2[e]).numpy()) < 1e-12


def test_forward_tokens_path_agrees():
    T, H, I, E, K = 40, 16, 8, 8, 3
    w = small(T, H, I, E, K, dtype="bf16")
    inp = make_inputs(w)
    ids, g, _ = make_routing(w)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    toks = np.array([0, 7, 39, 7])
    yr = oracle.forward_tokens(inp["x"], ids, g, inp["up_proj"], inp["down_proj"], toks)
    assert rel_err(yr, y[toks]) < 1e-13


def test_forward_t0():
    w = small(0, 8, 8, 4, 2)
    inp = make_inputs(w)
    y = oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                       inp["down_proj"])
    assert y.shape == (0, 8)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even (1 + 2^-6) wins.
    got = f32_from_bf16_bits(bf16_bits_from_f32(f))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.015625)
    assert got[3] == -2.5
    assert abs(got[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


# --------------------------------------------------------------------------- backward
def torch_backward(x, ids, g, W1, W2, dy):
    x, g, W1, W2 = [as64(a).requires_grad_(True) for a in (x, g, W1, W2)]
    y = brute_forward(x, ids, g, W1, W2)
    (y * as64(dy)).sum().backward()
    return x.grad.numpy(), W1.grad.numpy(), W2.grad.numpy(), g.grad.numpy()


@pytest.mark.parametrize("T,H,I,E,K,dtype,distinct", FWD_CASES)
def test_backward_matches_autograd(T, H, I, E, K, dtype, distinct):
    w = small(T, H, I, E, K, dtype=dtype)
    inp = make_inputs(w, with_dy=True)
    rng = np.random.default_rng(T * 77 + I)
    ids = random_ids(rng, T, K, E, distinct=distinct)
    g = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    got = oracle.backward(inp["dy"], inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    want = torch_backward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"], inp["dy"])
    for name, a, b in zip(("dx", "d_up", "d_down", "d_topk"), got, want):
        assert rel_err(a, b) < 1e-12, name


def test_backward_finite_differences():
    """Central differences of L = <dY, y(θ)> on the oracle's own forward (fp32 inputs;
    the step is the exact fp32 difference)."""
    T, H, I, E, K = 6, 8, 6, 3, 2
    w = small(T, H, I, E, K)
    inp = make_inputs(w, with_dy=True)
    rng = np.random.default_rng(9)
    ids = random_ids(rng, T, K, E, distinct=True)
    g = rng.uniform(0.2, 1.0, size=(T, K)).astype(np.float32)
    dy = inp["dy"].astype(np.float64)
    args = dict(x=inp["x"], g=g, up=inp["up_proj"], down=inp["down_proj"])
    dx, d_up, d_down, dg = oracle.backward(inp["dy"], inp["x"], ids, g, inp["up_proj"],
                                           inp["down_proj"])
    grads = dict(x=dx, g=dg, up=d_up, down=d_down)

    def L(a):
        return float((oracle.forward(a["x"], ids, a["g"], a["up"], a["down"]) * dy).sum())

    for name in ("x", "g", "up", "down"):
        flat_n = args[name].size
        for idx in rng.choice(flat_n, size=6, replace=False):
            ap, am = dict(args), dict(args)
            base = args[name].ravel()[idx]
            step = max(1e-3, 1e-3 * abs(float(base)))
            vp = args[name].copy()
            vm = args[name].copy()
            vp.ravel()[idx] = np.float32(base + step)
            vm.ravel()[idx] = np.float32(base - step)
            ap[name], am[name] = vp, vm
            fd = (L(ap) - L(am)) / (float(vp.ravel()[idx]) - float(vm.ravel()[idx]))
            an = grads[name].ravel()[idx]
            scale = np.abs(grads[name]).max()
            assert abs(fd - an) <= 1e-5 * scale + 1e-9, (name, idx, fd, an)


def test_backward_linearity_identities():
    """y is linear in the gates and in W2, so <dY, y> = Σ g·d_g = <W2, dW2>."""
    T, H, I, E, K = 25, 16, 12, 5, 3
    w = small(T, H, I, E, K, dtype="bf16")
    inp = make_inputs(w, with_dy=True)
    ids, g, _ = make_routing(w)
    y = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
    dx, d_up, d_down, dg = oracle.backward(inp["dy"], inp["x"], ids, g, inp["up_proj"],
                                           inp["down_proj"])
    dyv = f32_from_bf16_bits(inp["dy"]).astype(np.float64)
    W2 = f32_from_bf16_bits(inp["down_proj"]).astype(np.float64)
    lhs = float((dyv * y).sum())
    assert abs(lhs - float((g.astype(np.float64) * dg).sum())) < 1e-12 * max(1, abs(lhs)) * 100
    assert abs(lhs - float((W2 * d_down).sum())) < 1e-12 * max(1, abs(lhs)) * 100


def test_backward_empty_expert_grads_exactly_zero():
    T, H, I, E, K = 10, 8, 8, 4, 2
    w = small(T, H, I, E, K)
    inp = make_inputs(w, with_dy=True)
    ids = np.random.default_rng(4).choice([0, 2], size=(T, K)).astype(np.int32)
    g = np.full((T, K), 0.5, np.float32)
    _, d_up, d_down, _ = oracle.backward(inp["dy"], inp["x"], ids, g, inp["up_proj"],
                                         inp["down_proj"])
    assert not d_up[[1, 3]].any() and not d_down[[1, 3]].any()
    assert d_up[[0, 2]].any() and d_down[[0, 2]].any()


def test_backward_sampled_agrees_with_full():
    T, H, I, E, K = 18, 8, 6, 4, 2
    w = small(T, H, I, E, K, dtype="bf16")
    inp = make_inputs(w, with_dy=True)
    ids, g, _ = make_routing(w)
    dx, d_up, d_down, dg = oracle.backward(inp["dy"], inp["x"], ids, g, inp["up_proj"],
                                           inp["down_proj"])
    toks = [0, 5, 17]
    w1c = [(0, 0), (1, 7), (3, 11), (2, 5)]
    w2r = [(0, 0), (3, 5), (1, 2)]
    sx, sg, s1, s2 = oracle.backward_sampled(inp["dy"], inp["x"], ids, g, inp["up_proj"],
                                             inp["down_proj"], toks, w1c, w2r)
    assert rel_err(sx, dx[toks]) < 1e-12
    assert rel_err(sg, dg[toks]) < 1e-12
    assert rel_err(s1, np.stack([d_up[e][:, j] for e, j in w1c])) < 1e-12
    assert rel_err(s2, np.stack([d_down[e][i, :] for e, i in w2r])) < 1e-12


# --------------------------------------------------------------------------- shared expert
# Issue page, section 6.1, and the EP overlap issue, section 4.3: the shared
# expert's SwiGLU FFN output is added to the combined routed output.
def dense_ffn(x, W1, W2):
    Is = W2.shape[0]
    h = x @ W1
    return (F.silu(h[:, :Is]) * h[:, Is:]) @ W2


def shared_inputs(T=9, H=16, I=8, E=3, K=2, Is=24, dtype="f32", cfg_id=140):
    w = small(T, H, I, E, K, dtype=dtype, cfg_id=cfg_id, Is=Is)
    return make_inputs(w, with_dy=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_expert_is_dense_swiglu_ffn(dtype):
    """The shared term against torch.nn.functional.silu and plain matmuls."""
    inp = shared_inputs(dtype=dtype)
    got = oracle.shared_expert(inp["x"], inp["shared_up"], inp["shared_down"])
    want = dense_ffn(as64(inp["x"]), as64(inp["shared_up"]), as64(inp["shared_down"]))
    assert rel_err(got, want.numpy()) < 1e-12


def test_forward_shared_with_zero_shared_weights_is_the_routed_layer():
    inp = shared_inputs()
    zup, zdown = np.zeros_like(inp["shared_up"]), np.zeros_like(inp["shared_down"])
    got = oracle.forward_shared(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                                inp["down_proj"], zup, zdown)
    want = oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                          inp["down_proj"])
    assert np.array_equal(got, want)


def test_shared_term_does_not_depend_on_the_routing():
    inp = shared_inputs()
    rng = np.random.default_rng(3)
    diffs = []
    for _ in range(2):
        ids = random_ids(rng, 9, 2, 3)
        g = rng.uniform(0.1, 1.0, size=(9, 2)).astype(np.float32)
        a = oracle.forward_shared(inp["x"], ids, g, inp["up_proj"], inp["down_proj"],
                                  inp["shared_up"], inp["shared_down"])
        b = oracle.forward(inp["x"], ids, g, inp["up_proj"], inp["down_proj"])
        diffs.append(a - b)
    assert rel_err(diffs[0], diffs[1]) < 1e-12


def test_shared_expert_splits_into_chunks_of_the_routed_width():
    """Is = 3I: the shared FFN equals the sum of three width-I SwiGLU FFNs whose gate
    columns are gate chunk c, up columns up chunk c and down rows chunk c (the
    decomposition the GPU schedules as three extra experts)."""
    I, Is = 8, 24
    inp = shared_inputs(I=I, Is=Is)
    W1, W2 = inp["shared_up"], inp["shared_down"]
    whole = oracle.shared_expert(inp["x"], W1, W2)
    parts = 0.0
    for c in range(Is // I):
        w1c = np.concatenate([W1[:, c * I:(c + 1) * I], W1[:, Is + c * I:Is + (c + 1) * I]], axis=1)
        parts = parts + oracle.shared_expert(inp["x"], np.ascontiguousarray(w1c),
                                             np.ascontiguousarray(W2[c * I:(c + 1) * I]))
    assert rel_err(parts, whole) < 1e-12


def test_backward_shared_matches_autograd():
    inp = shared_inputs()
    got = oracle.backward_shared(inp["dy"], inp["x"], inp["topk_ids"], inp["topk_weights"],
                                 inp["up_proj"], inp["down_proj"], inp["shared_up"],
                                 inp["shared_down"])
    x, g, W1, W2, S1, S2 = [as64(a).requires_grad_(True) for a in
                            (inp["x"], inp["topk_weights"], inp["up_proj"], inp["down_proj"],
                             inp["shared_up"], inp["shared_down"])]
    y = brute_forward(x, inp["topk_ids"], g, W1, W2) + dense_ffn(x, S1, S2)
    (y * as64(inp["dy"])).sum().backward()
    want = (x.grad, W1.grad, W2.grad, g.grad, S1.grad, S2.grad)
    for name, a, b in zip(("dx", "d_up", "d_down", "d_topk", "d_shared_up", "d_shared_down"),
                          got, want):
        assert rel_err(a, b.numpy()) < 1e-12, name


def test_forward_shared_t0():
    inp = shared_inputs(T=0)
    y = oracle.forward_shared(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                              inp["down_proj"], inp["shared_up"], inp["shared_down"])
    assert y.shape == (0, 16)
