"""The shared expert against the oracle (forward and backward).

Issue page, section 6.1 ("shared-expert fused MoE"): an optional shared
expert whose SwiGLU FFN runs alongside the routed experts and whose output the
combine adds.  The kernels run it as Is / I extra experts (column and row
chunks of its weights) that every token reaches with gate 1.  Tolerances as
for the routed layer: max|err| / max|ref| <= 1e-2 (bf16), 1e-5 (fp32).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

FWD = [
    # name, T, H, I, E, K, Is, dtype, routing
    ("sh_fast_s1", 600, 512, 256, 8, 3, 256, "bf16", "uniform"),
    ("sh_fast_s2_bm64", 120, 256, 128, 16, 2, 256, "bf16", "uniform"),
    ("sh_engine_s2", 333, 264, 200, 6, 2, 400, "bf16", "uniform"),
    ("sh_zipf_empty", 515, 256, 128, 16, 4, 384, "bf16", "zipf"),
    ("sh_one_token", 1, 256, 128, 8, 2, 128, "bf16", "uniform"),
    ("sh_f32", 256, 256, 128, 8, 2, 256, "f32", "uniform"),
]
BWD = [
    ("shb_fast_s1", 600, 512, 256, 8, 3, 256, "uniform"),
    ("shb_fast_s3", 300, 256, 128, 16, 2, 384, "uniform"),
    ("shb_engine_s2", 333, 264, 200, 6, 2, 400, "uniform"),
    ("shb_zipf_empty", 515, 256, 128, 16, 4, 256, "zipf"),
]


def workload(name, seed, T, H, I, E, K, Is, dtype="bf16", routing="uniform"):
    return Workload(name, seed, T=T, H=H, I=I, E=E, K=K, Is=Is, dtype=dtype, routing=routing,
                    n_empty=3 if routing == "zipf" else 0)


def fwd(gpu_lib, d, **kw):
    return gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], shared_up_proj_weight=d["shared_up"],
                               shared_down_proj_weight=d["shared_down"], **kw)


@pytest.mark.parametrize("case", FWD, ids=[c[0] for c in FWD])
def test_shared_forward_parity(gpu_lib, case):
    name, T, H, I, E, K, Is, dtype, routing = case
    inp = make_inputs(workload(name, 600 + FWD.index(case), T, H, I, E, K, Is, dtype, routing))
    say(f"[shared] case={name} T={T} H={H} I={I} E={E} K={K} Is={Is}")
    y = fwd(gpu_lib, to_device(inp))
    torch.cuda.synchronize()
    ref = oracle.forward_shared(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                                inp["down_proj"], inp["shared_up"], inp["shared_down"])
    err = max_rel_err(host_f64(y), ref)
    say(f"[shared] case={name} max_rel_err={err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("case", BWD, ids=[c[0] for c in BWD])
def test_shared_backward_parity(gpu_lib, case):
    name, T, H, I, E, K, Is, routing = case
    inp = make_inputs(workload(name, 620 + BWD.index(case), T, H, I, E, K, Is, "bf16", routing),
                      with_dy=True)
    d = to_device(inp)
    say(f"[shared-bwd] case={name} T={T} H={H} I={I} E={E} K={K} Is={Is}")
    _, saved = fwd(gpu_lib, d, save_for_backward=True)
    grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], saved, shared_up_proj_weight=d["shared_up"],
                                shared_down_proj_weight=d["shared_down"])
    torch.cuda.synchronize()
    ref = oracle.backward_shared(inp["dy"], inp["x"], inp["topk_ids"], inp["topk_weights"],
                                 inp["up_proj"], inp["down_proj"], inp["shared_up"],
                                 inp["shared_down"])
    names = ("dx", "d_up", "d_down", "d_topk", "d_shared_up", "d_shared_down")
    errs = {n: max_rel_err(host_f64(g), r) for n, g, r in zip(names, grads, ref)}
    say(f"[shared-bwd] case={name} " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_shared_weights_reproduce_the_routed_layer(gpu_lib, dtype):
    inp = make_inputs(workload("sh_zero", 640, 300, 256, 128, 8, 2, 256, dtype))
    d = to_device(inp)
    d["shared_up"].zero_()
    d["shared_down"].zero_()
    say(f"[shared] zero shared weights {dtype}")
    y_s = fwd(gpu_lib, d)
    y = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                            d["down_proj"])
    torch.cuda.synchronize()
    assert torch.equal(y_s, y)


def test_pipeline_flag_with_shared_expert_runs_the_bulk_launches(gpu_lib):
    inp = make_inputs(workload("sh_pipe", 641, 400, 512, 256, 8, 2, 256))
    d = to_device(inp)
    say("[shared] pipelined flag")
    y_p = fwd(gpu_lib, d, pipelined=True)
    y_b = fwd(gpu_lib, d)
    torch.cuda.synchronize()
    assert torch.equal(y_p, y_b)


def test_shared_with_zero_tokens(gpu_lib):
    inp = make_inputs(workload("sh_t0", 642, 0, 256, 128, 4, 2, 256), with_dy=True)
    d = to_device(inp)
    say("[shared] T=0")
    y, saved = fwd(gpu_lib, d, save_for_backward=True)
    grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], saved, shared_up_proj_weight=d["shared_up"],
                                shared_down_proj_weight=d["shared_down"])
    torch.cuda.synchronize()
    assert y.shape == (0, 256)
    for g in grads[1:3] + grads[4:]:
        assert not g.float().abs().sum().item()


def test_shared_forward_prefill_size_sampled(gpu_lib):
    w = WORKLOADS["prefill_shared_bf16"]
    say("[shared-full] generating prefill_shared_bf16 (Is = 2I)")
    inp = make_inputs(w)
    d = to_device(inp)
    say("[shared-full] running")
    y = fwd(gpu_lib, d)
    torch.cuda.synchronize()
    toks = np.random.default_rng(5).choice(w.T, size=16, replace=False)
    ref = (oracle.forward_tokens(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                                 inp["down_proj"], toks)
           + oracle.shared_expert(inp["x"][toks], inp["shared_up"], inp["shared_down"]))
    err = max_rel_err(host_f64(y[torch.from_numpy(toks).cuda()]), ref)
    say(f"[shared-full] sampled 16 tokens max_rel_err={err:.3e}")
    assert err <= TOL["bf16"]


def test_shared_backward_full_size_sampled(gpu_lib):
    # the forward+backward shape with Is = I; every gradient on sampled rows or
    # columns (the shared part is the routed definition at one expert, gate 1)
    w = WORKLOADS["fwdbwd_shared_bf16"]
    say("[shared-bwd-full] generating fwdbwd_shared_bf16")
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    say(f"[shared-bwd-full] running T={w.T} H={w.H} I={w.I} E={w.E} K={w.K} Is={w.Is}")
    _, saved = fwd(gpu_lib, d, save_for_backward=True)
    dx, d_up, d_down, d_topk, ds_up, ds_down = gpu_lib.moe_ffn_bwd(
        d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"], d["down_proj"], saved,
        shared_up_proj_weight=d["shared_up"], shared_down_proj_weight=d["shared_down"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 10, replace=False)]))
    w1c = [(int(rng.integers(w.E)), int(j)) for j in [0, w.I, 2 * w.I - 1]]
    w2r = [(int(rng.integers(w.E)), int(i)) for i in [0, w.I - 1]]
    rx, rg, r1, r2 = oracle.backward_sampled(inp["dy"], inp["x"], inp["topk_ids"],
                                             inp["topk_weights"], inp["up_proj"],
                                             inp["down_proj"], toks, w1c, w2r)
    sc = [0, w.Is - 1, w.Is, 2 * w.Is - 1] + [int(j) for j in rng.choice(2 * w.Is, 4)]
    sr = [0, w.Is - 1] + [int(i) for i in rng.choice(w.Is, 4)]
    ids1 = np.zeros((w.T, 1), np.int32)
    g1 = np.ones((w.T, 1), np.float32)
    sx, _, s1, s2 = oracle.backward_sampled(inp["dy"], inp["x"], ids1, g1,
                                            inp["shared_up"][None], inp["shared_down"][None],
                                            toks, [(0, j) for j in sc], [(0, i) for i in sr])
    tk = torch.from_numpy(toks).cuda()
    errs = dict(
        dx=max_rel_err(host_f64(dx[tk]), rx + sx),
        d_topk=max_rel_err(d_topk[tk].double().cpu().numpy(), rg),
        d_up=max_rel_err(np.stack([host_f64(d_up[e, :, j]) for e, j in w1c]), r1),
        d_down=max_rel_err(np.stack([host_f64(d_down[e, i, :]) for e, i in w2r]), r2),
        d_shared_up=max_rel_err(np.stack([host_f64(ds_up[:, j]) for j in sc]), s1),
        d_shared_down=max_rel_err(np.stack([host_f64(ds_down[i, :]) for i in sr]), s2))
    say("[shared-bwd-full] " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


def test_shared_backward_rejects_a_routed_only_saved_context(gpu_lib):
    # the saved context of the same batch's forward without the shared expert
    # (its problem hash differs in Is), padded to the shared layout's size
    inp = make_inputs(workload("sh_foreign", 643, 300, 256, 128, 8, 2, 256), with_dy=True)
    d = to_device(inp)
    say("[shared] routed-only saved context")
    _, saved_s = fwd(gpu_lib, d, save_for_backward=True)
    _, saved_r = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                     d["down_proj"], save_for_backward=True)
    foreign = torch.zeros_like(saved_s)
    foreign[:saved_r.numel()] = saved_r
    torch.cuda.synchronize()
    args = (d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"], d["down_proj"])
    sh = dict(shared_up_proj_weight=d["shared_up"], shared_down_proj_weight=d["shared_down"])
    with pytest.raises(gpu_lib.MoEFFNError) as ei:
        gpu_lib.moe_ffn_bwd(*args, foreign, check_saved=True, **sh)
    assert ei.value.status == 7
    *grads, ws = gpu_lib.moe_ffn_bwd(*args, foreign, return_ws=True, **sh)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == gpu_lib.DEV_BAD_SAVED
    assert len(grads) == 6
    for g in grads:
        assert not g.float().abs().sum().item()
