"""The backward split into its data half and its weight half.

EP overlap issue, section 2.3 "W/D split + deferred W queue" and section 4.5's
interface draft: a D-only call that yields the input gradient and a W-only
call that a scheduler may run later.  moe_ffn_bwd_d followed by moe_ffn_bwd_w
must match the oracle's backward (element by element on small shapes, with
Zipf routing that leaves experts empty; sampled at full size) and reproduce
moe_ffn_bwd bit for bit; a weight half given a workspace that does not hold
the data half of the same saved context must read nothing from it and report
so.  Tolerance: max|err| / max|ref| <= 1e-2 per gradient.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, I, E, K, routing
    ("split_tiles", 600, 512, 384, 8, 3, "uniform"),
    ("split_ragged", 333, 264, 200, 6, 2, "uniform"),
    ("split_zipf_empty", 515, 256, 128, 16, 4, "zipf"),
    ("split_one_token", 1, 256, 128, 8, 2, "uniform"),
]


def fwd_saved(gpu_lib, d):
    return gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], save_for_backward=True)[1]


def split(gpu_lib, d, saved, **kw):
    dx, d_topk, ws = gpu_lib.moe_ffn_bwd_d(d["dy"], d["topk_ids"], d["topk_weights"],
                                           d["up_proj"], d["down_proj"], saved)
    d_up, d_down = gpu_lib.moe_ffn_bwd_w(d["dy"], d["x"], d["topk_ids"], d["up_proj"],
                                         d["down_proj"], saved, ws, **kw)
    return (dx, d_up, d_down, d_topk), ws


def whole(gpu_lib, d, saved):
    return gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], saved)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle(gpu_lib, case):
    name, T, H, I, E, K, routing = case
    w = Workload(name, 500 + CASES.index(case), T=T, H=H, I=I, E=E, K=K, routing=routing,
                 n_empty=3 if routing == "zipf" else 0)
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    say(f"[split-oracle] case={name} T={T} H={H} I={I} E={E} K={K}")
    saved = fwd_saved(gpu_lib, d)
    got, ws = split(gpu_lib, d, saved)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    refs = oracle.backward(inp["dy"], inp["x"], inp["topk_ids"], inp["topk_weights"],
                           inp["up_proj"], inp["down_proj"])
    for g, r, n in zip(got, refs, ("dx", "d_up", "d_down", "d_topk")):
        e = max_rel_err(host_f64(g), r)
        say(f"[split-oracle] case={name} {n} max_rel_err={e:.3e}")
        assert e <= TOL["bf16"], (n, e)


def test_split_sampled_full_size_vs_oracle(gpu_lib):
    w = WORKLOADS["fwdbwd_bf16"]
    say("[split-oracle-full] generating fwdbwd_bf16")
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    say("[split-oracle-full] running")
    saved = fwd_saved(gpu_lib, d)
    (dx, d_up, d_down, d_topk), ws = split(gpu_lib, d, saved)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 14, replace=False)]))
    w1c = [(int(rng.integers(w.E)), int(j)) for j in
           np.concatenate([[0, w.I - 1, w.I, 2 * w.I - 1], rng.choice(2 * w.I, 10)])]
    w2r = [(int(rng.integers(w.E)), int(i)) for i in
           np.concatenate([[0, w.I - 1], rng.choice(w.I, 10)])]
    rx, rg, r1, r2 = oracle.backward_sampled(inp["dy"], inp["x"], inp["topk_ids"],
                                             inp["topk_weights"], inp["up_proj"],
                                             inp["down_proj"], toks, w1c, w2r)
    tk = torch.from_numpy(toks).cuda()
    errs = dict(dx=max_rel_err(host_f64(dx[tk]), rx),
                d_topk=max_rel_err(d_topk[tk].double().cpu().numpy(), rg),
                d_up=max_rel_err(np.stack([host_f64(d_up[e, :, j]) for e, j in w1c]), r1),
                d_down=max_rel_err(np.stack([host_f64(d_down[e, i, :]) for e, i in w2r]), r2))
    say("[split-oracle-full] " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_equals_whole(gpu_lib, case):
    name, T, H, I, E, K, routing = case
    w = Workload(name, 500 + CASES.index(case), T=T, H=H, I=I, E=E, K=K, routing=routing,
                 n_empty=3 if routing == "zipf" else 0)
    d = to_device(make_inputs(w, with_dy=True))
    say(f"[split] case={name} T={T} H={H} I={I} E={E} K={K}")
    saved = fwd_saved(gpu_lib, d)
    got, ws = split(gpu_lib, d, saved)
    ref = whole(gpu_lib, d, saved)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    for g, r, n in zip(got, ref, ("dx", "d_up", "d_down", "d_topk")):
        assert torch.equal(g, r), n


def test_split_equals_whole_full_size(gpu_lib):
    w = WORKLOADS["fwdbwd_bf16"]
    say("[split-full] generating fwdbwd_bf16")
    d = to_device(make_inputs(w, with_dy=True))
    say("[split-full] running")
    saved = fwd_saved(gpu_lib, d)
    got, ws = split(gpu_lib, d, saved)
    ref = whole(gpu_lib, d, saved)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    for g, r, n in zip(got, ref, ("dx", "d_up", "d_down", "d_topk")):
        assert torch.equal(g, r), n


def test_weight_half_rejects_a_workspace_of_another_forward(gpu_lib):
    w = Workload("split_other", 520, T=256, H=256, I=128, E=8, K=2)
    d = to_device(make_inputs(w, with_dy=True))
    say("[split] workspace of another forward")
    saved_a = fwd_saved(gpu_lib, d)
    saved_b = fwd_saved(gpu_lib, d)  # same inputs, a different forward call
    _, _, ws_a = gpu_lib.moe_ffn_bwd_d(d["dy"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                       d["down_proj"], saved_a)
    d_up, d_down = gpu_lib.moe_ffn_bwd_w(d["dy"], d["x"], d["topk_ids"], d["up_proj"],
                                         d["down_proj"], saved_b, ws_a)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws_a) == gpu_lib.DEV_BAD_WS
    assert not d_up.float().abs().sum().item() and not d_down.float().abs().sum().item()
    # the host-side check refuses it before launching anything
    with pytest.raises(gpu_lib.MoEFFNError):
        gpu_lib.moe_ffn_bwd_w(d["dy"], d["x"], d["topk_ids"], d["up_proj"], d["down_proj"],
                              saved_b, ws_a, check_saved=True)
    # and the right pairing still works on the same buffers
    got, ws = split(gpu_lib, d, saved_b)
    ref = whole(gpu_lib, d, saved_b)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_weight_half_rejects_a_workspace_without_data_half(gpu_lib):
    w = Workload("split_fresh", 521, T=128, H=256, I=128, E=4, K=2)
    d = to_device(make_inputs(w, with_dy=True))
    say("[split] zeroed workspace")
    saved = fwd_saved(gpu_lib, d)
    _, _, ws = gpu_lib.moe_ffn_bwd_d(d["dy"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                     d["down_proj"], saved)
    ws.zero_()
    d_up, d_down = gpu_lib.moe_ffn_bwd_w(d["dy"], d["x"], d["topk_ids"], d["up_proj"],
                                         d["down_proj"], saved, ws)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == gpu_lib.DEV_BAD_WS
    assert not d_up.float().abs().sum().item() and not d_down.float().abs().sum().item()


def test_split_with_zero_tokens(gpu_lib):
    w = Workload("split_zero", 522, T=0, H=256, I=128, E=4, K=2)
    d = to_device(make_inputs(w, with_dy=True))
    say("[split] T=0")
    saved = fwd_saved(gpu_lib, d)
    dx, d_topk, ws = gpu_lib.moe_ffn_bwd_d(d["dy"], d["topk_ids"], d["topk_weights"],
                                           d["up_proj"], d["down_proj"], saved)
    d_up, d_down = gpu_lib.moe_ffn_bwd_w(d["dy"], d["x"], d["topk_ids"], d["up_proj"],
                                         d["down_proj"], saved, ws)
    torch.cuda.synchronize()
    assert dx.shape == (0, 256) and d_topk.shape == (0, 2)
    assert not d_up.float().abs().sum().item() and not d_down.float().abs().sum().item()
