"""Backward parity of the HIP path against the CPU oracle.

HyperMegaMoE issue page, section 2.2 "backward fusion": given dY the call
returns dx, d_up_proj_weight, d_down_proj_weight and d_topk_weights (topk_ids
gets none).  Small shapes are compared in full; the forward+backward workload
at full size on sampled rows and columns that the oracle computes one by one.
Tolerance: max|g - g_ref| / max|g_ref| <= 1e-2 per gradient (bf16).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

SMALL = [
    # name, T, H, I, E, K, routing
    ("bwd_tiles", 600, 512, 384, 8, 3, "uniform"),
    ("bwd_ragged", 333, 264, 200, 6, 2, "uniform"),
    ("bwd_zipf_empty", 515, 256, 128, 16, 4, "zipf"),
    ("bwd_dups", 129, 128, 64, 4, 3, "replace"),
    ("bwd_one_token", 1, 256, 128, 8, 2, "uniform"),
    ("bwd_wide_k", 150, 384, 136, 5, 5, "uniform"),
    # 8 rows per expert: the saving forward runs the pipelined launch by default
    ("bwd_decode_like", 64, 512, 256, 32, 4, "uniform"),
    # the largest K (the dx combine sums 32 rows in four rounds of 8; 32
    # d_topk lanes per token)
    ("bwd_k32", 40, 256, 128, 64, 32, "uniform"),
    # the largest E: about 2 rows per expert, most experts empty (their weight
    # gradients must come out as exact zeros)
    ("bwd_many_experts", 300, 256, 128, 1024, 8, "uniform"),
]
NAMES = ("dx", "d_up", "d_down", "d_topk")


def run(gpu_lib, inp):
    d = to_device(inp)
    y, saved = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                   d["down_proj"], save_for_backward=True)
    grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], saved)
    torch.cuda.synchronize()
    return y, grads


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_full_parity_small(gpu_lib, case):
    name, T, H, I, E, K, routing = case
    w = Workload(name, 300 + SMALL.index(case), T=T, H=H, I=I, E=E, K=K, routing=routing,
                 n_empty=3 if routing == "zipf" else 0)
    inp = make_inputs(w, with_dy=True)
    say(f"[bwd] case={name} T={T} H={H} I={I} E={E} K={K}")
    _, grads = run(gpu_lib, inp)
    ref = oracle.backward(inp["dy"], inp["x"], inp["topk_ids"], inp["topk_weights"],
                          inp["up_proj"], inp["down_proj"])
    errs = {n: max_rel_err(host_f64(g), r) for n, g, r in zip(NAMES, grads, ref)}
    say(f"[bwd] case={name} " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
    counts = np.bincount(inp["topk_ids"].ravel(), minlength=E)
    empty = np.where(counts == 0)[0]
    if routing == "zipf":
        assert len(empty) >= 3
    if len(empty):
        # experts without rows get exact zeros, not merely small values
        assert not grads[1][empty].float().abs().sum().item()
        assert not grads[2][empty].float().abs().sum().item()


def test_bwd_sampled_parity_full_size(gpu_lib):
    w = WORKLOADS["fwdbwd_bf16"]
    say("[bwd-full] generating fwdbwd_bf16")
    inp = make_inputs(w, with_dy=True)
    say(f"[bwd-full] running T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    _, (dx, d_up, d_down, d_topk) = run(gpu_lib, inp)
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 14, replace=False)]))
    w1c = [(int(rng.integers(w.E)), int(j)) for j in
           np.concatenate([[0, w.I - 1, w.I, 2 * w.I - 1], rng.choice(2 * w.I, 10)])]
    w2r = [(int(rng.integers(w.E)), int(i)) for i in
           np.concatenate([[0, w.I - 1], rng.choice(w.I, 10)])]
    rx, rg, r1, r2 = oracle.backward_sampled(inp["dy"], inp["x"], inp["topk_ids"],
                                             inp["topk_weights"], inp["up_proj"],
                                             inp["down_proj"], toks, w1c, w2r)
    tk = torch.from_numpy(toks).cuda()
    got_dx = host_f64(dx[tk])
    got_dg = d_topk[tk].double().cpu().numpy()
    got_1 = np.stack([host_f64(d_up[e, :, j]) for e, j in w1c])
    got_2 = np.stack([host_f64(d_down[e, i, :]) for e, i in w2r])
    errs = dict(dx=max_rel_err(got_dx, rx), d_topk=max_rel_err(got_dg, rg),
                d_up=max_rel_err(got_1, r1), d_down=max_rel_err(got_2, r2))
    say("[bwd-full] " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
    for t in (dx, d_up, d_down, d_topk):
        assert torch.isfinite(t.float()).all()


def test_bwd_is_deterministic(gpu_lib):
    w = Workload("bdet", 320, T=700, H=256, I=192, E=8, K=3)
    inp = make_inputs(w, with_dy=True)
    say("[bwd] determinism")
    _, g1 = run(gpu_lib, inp)
    _, g2 = run(gpu_lib, inp)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_zero_tokens_zeroes_weight_grads(gpu_lib):
    w = Workload("b0", 321, T=0, H=128, I=64, E=4, K=2)
    inp = make_inputs(w, with_dy=True)
    say("[bwd] T=0")
    _, (dx, d_up, d_down, d_topk) = run(gpu_lib, inp)
    assert dx.shape == (0, 128) and d_topk.shape == (0, 2)
    assert not d_up.float().abs().sum().item() and not d_down.float().abs().sum().item()


def test_autograd_matches_direct_call(gpu_lib):
    w = Workload("bag", 322, T=200, H=256, I=128, E=8, K=2)
    inp = make_inputs(w, with_dy=True)
    say("[bwd] autograd")
    d = to_device(inp)
    _, (dx, d_up, d_down, d_topk) = run(gpu_lib, inp)
    x = d["x"].clone().requires_grad_(True)
    g = d["topk_weights"].clone().requires_grad_(True)
    up = d["up_proj"].clone().requires_grad_(True)
    down = d["down_proj"].clone().requires_grad_(True)
    y = gpu_lib.moe_ffn(x, d["topk_ids"], g, up, down)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    assert torch.equal(x.grad, dx) and torch.equal(up.grad, d_up)
    assert torch.equal(down.grad, d_down) and torch.equal(g.grad, d_topk)


def test_bwd_rejects_fp32(gpu_lib):
    w = Workload("bf32", 323, T=8, H=64, I=32, E=2, K=1, dtype="f32")
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    _, saved = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                   d["down_proj"], save_for_backward=True)
    with pytest.raises(gpu_lib.MoEFFNError) as ei:
        gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                            d["down_proj"], saved)
    assert ei.value.status == 3


def test_bwd_checks_the_saved_context(gpu_lib):
    # a saved context written by the forward of another problem (T = 200) but
    # big enough for this one (T = 300)
    wa = Workload("bsa", 324, T=200, H=256, I=128, E=8, K=2)
    wb = Workload("bsb", 325, T=300, H=256, I=128, E=8, K=2)
    da, db = to_device(make_inputs(wa, with_dy=True)), to_device(make_inputs(wb, with_dy=True))
    say("[bwd] foreign saved context")
    _, saved_b = gpu_lib.moe_ffn_fwd(db["x"], db["topk_ids"], db["topk_weights"], db["up_proj"],
                                     db["down_proj"], save_for_backward=True)
    _, saved_a = gpu_lib.moe_ffn_fwd(da["x"], da["topk_ids"], da["topk_weights"], da["up_proj"],
                                     da["down_proj"], save_for_backward=True)
    foreign = torch.zeros_like(saved_b)
    foreign[:saved_a.numel()] = saved_a
    torch.cuda.synchronize()
    args = (db["dy"], db["x"], db["topk_ids"], db["topk_weights"], db["up_proj"], db["down_proj"])
    with pytest.raises(gpu_lib.MoEFFNError) as ei:
        gpu_lib.moe_ffn_bwd(*args, foreign, check_saved=True)
    assert ei.value.status == 7
    # without the host check: nothing faults, all outputs are zero, the status says why
    *grads, ws = gpu_lib.moe_ffn_bwd(*args, foreign, return_ws=True)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == gpu_lib.DEV_BAD_SAVED
    for g in grads:
        assert not g.float().abs().sum().item()
    # the matching context passes both checks and the status is clean
    *grads, ws = gpu_lib.moe_ffn_bwd(*args, saved_b, check_saved=True, return_ws=True)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    assert grads[1].float().abs().sum().item() > 0
