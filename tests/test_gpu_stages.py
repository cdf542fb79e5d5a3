"""Stage-by-stage parity and stability of the HIP path.

* Stages (overlap explainer page, section 6: a pipelined operator is checked
  against the plain stage sequence one stage at a time): after an inference
  forward the routing arrays left in the workspace equal the oracle's bit for
  bit, and act and o (rows in permuted order) match the oracle's intermediates
  within the tolerance, on every forward kernel family and in the pipelined
  launch.
* Consecutive calls (HyperMegaMoE issue page, section 7.3: repeated
  iterations must leave no residue and must not pollute one another): one
  workspace filled with 0xFF, reused by alternating configurations for 48
  calls, gives each configuration its own first result bit for bit.
* Interleaving (issue page, section 7.1: several forwards, then the
  backward): fwd(A), fwd(B), bwd(B), bwd(A) with separate saved contexts and
  one backward workspace give each pair's gradients bit for bit.
* Token-dimension tails (issue page, section 7.2): the skewed workload at
  T = 8191, sampled.
Tolerance: max|err| / max|ref| <= 1e-2 (bf16), 1e-5 (fp32).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

STAGE_CASES = [
    # name, T, H, I, E, K, dtype, routing, flags
    ("bm64", 40, 512, 256, 16, 4, "bf16", "uniform", 0),
    ("bm128", 600, 512, 384, 8, 3, "bf16", "uniform", 0),
    ("bm128_big_gemm2", 1000, 512, 256, 8, 3, "bf16", "uniform", 0),
    ("big_tiles", 1100, 512, 256, 4, 2, "bf16", "uniform", 0),
    ("zipf_empty", 515, 256, 128, 16, 4, "bf16", "zipf", 0),
    ("engine_ragged", 333, 264, 200, 6, 2, "bf16", "uniform", 0),
    ("f32", 77, 136, 72, 5, 3, "f32", "uniform", 0),
    ("pipelined", 700, 512, 384, 8, 3, "bf16", "uniform", 2),
]


@pytest.mark.parametrize("case", STAGE_CASES, ids=[c[0] for c in STAGE_CASES])
def test_stages_match_oracle_intermediates(gpu_lib, case):
    name, T, H, I, E, K, dtype, routing, flags = case
    w = Workload(name, 900 + STAGE_CASES.index(case), T=T, H=H, I=I, E=E, K=K, dtype=dtype,
                 routing=routing, n_empty=3 if routing == "zipf" else 0)
    inp = make_inputs(w)
    d = to_device(inp)
    say(f"[stages] case={name} T={T} H={H} I={I} E={E} K={K} {dtype} flags={flags}")
    y, ws = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], return_ws=True, flags=flags)
    torch.cuda.synchronize()
    st = gpu_lib.fwd_stages(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"], ws, flags)
    y_ref, mid = oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                                inp["down_proj"], intermediates=True)
    for k in ("counts", "offsets", "sorted_slot", "slot_pos"):
        assert np.array_equal(st[k].cpu().numpy(), mid[k]), k
    errs = dict(act=max_rel_err(host_f64(st["act"]), mid["act"]),
                o=max_rel_err(host_f64(st["o"]), mid["o"]),
                y=max_rel_err(host_f64(y), y_ref))
    say(f"[stages] case={name} " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)


POISON_CONFIGS = [
    # name, T, H, I, E, K, flags: 128-row tiles, 64-row tiles, the pipelined
    # launch, GEMM2 on 256-row tiles, and the last one on 16 workgroups, where
    # both GEMMs hand out their last rounds by tickets (counters that routing
    # must reset on every call)
    ("p_bm128", 300, 256, 128, 8, 2, 0),
    ("p_bm64", 64, 256, 128, 16, 2, 0),
    ("p_pipe", 300, 256, 128, 8, 2, 2),
    ("p_big_gemm2", 1200, 256, 128, 8, 2, 0),
    ("p_ticketed_tails", 1300, 2048, 384, 7, 2, 0x200),
]


def test_poisoned_workspace_shared_by_alternating_calls(gpu_lib):
    cfgs = []
    for i, (name, T, H, I, E, K, flags) in enumerate(POISON_CONFIGS):
        w = Workload(name, 920 + i, T=T, H=H, I=I, E=E, K=K)
        inp = make_inputs(w)
        d = to_device(inp)
        say(f"[poison] reference {name}")
        y = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], flags=flags)
        torch.cuda.synchronize()
        ref = oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                             inp["down_proj"])
        assert max_rel_err(host_f64(y), ref) <= TOL["bf16"], name
        prob = gpu_lib.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"])
        cfgs.append((name, d, flags, y, gpu_lib.fwd_workspace_size(prob, flags)[0]))
    ws = torch.full((max(c[4] for c in cfgs),), 0xFF, dtype=torch.uint8, device="cuda")
    say("[poison] 48 alternating calls on one 0xFF workspace")
    for it in range(48):
        name, d, flags, y_ref, _ = cfgs[it % len(cfgs)]
        y = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], ws=ws, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {it} ({name}) differs from its first result"
        assert gpu_lib.read_status(ws) == 0


def _pair(gpu_lib, name, seed, T, H, I, E, K):
    w = Workload(name, seed, T=T, H=H, I=I, E=E, K=K)
    return to_device(make_inputs(w, with_dy=True))


def _fwd(gpu_lib, d):
    return gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], save_for_backward=True)


def _bwd(gpu_lib, d, saved, ws=None):
    return gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], saved, ws=ws)


def test_forwards_then_backwards_interleaved(gpu_lib):
    da = _pair(gpu_lib, "il_a", 930, 400, 256, 128, 8, 2)
    db = _pair(gpu_lib, "il_b", 931, 257, 256, 128, 8, 3)
    say("[interleave] references: fwd(A) bwd(A); fwd(B) bwd(B)")
    ya, sa = _fwd(gpu_lib, da)
    ga = _bwd(gpu_lib, da, sa)
    yb, sb = _fwd(gpu_lib, db)
    gb = _bwd(gpu_lib, db, sb)
    torch.cuda.synchronize()
    say("[interleave] fwd(A) fwd(B) bwd(B) bwd(A), one backward workspace")
    prob_a = gpu_lib.make_problem(da["x"], da["topk_ids"], da["up_proj"], da["down_proj"])
    prob_b = gpu_lib.make_problem(db["x"], db["topk_ids"], db["up_proj"], db["down_proj"])
    bws = torch.empty(max(gpu_lib.bwd_workspace_size(prob_a), gpu_lib.bwd_workspace_size(prob_b)),
                      dtype=torch.uint8, device="cuda")
    ya2, sa2 = _fwd(gpu_lib, da)
    yb2, sb2 = _fwd(gpu_lib, db)
    gb2 = _bwd(gpu_lib, db, sb2, ws=bws)
    ga2 = _bwd(gpu_lib, da, sa2, ws=bws)
    torch.cuda.synchronize()
    assert torch.equal(ya2, ya) and torch.equal(yb2, yb)
    for r, g, n in zip(ga + gb, ga2 + gb2, ("dx", "d_up", "d_down", "d_topk") * 2):
        assert torch.equal(r, g), n


def test_skewed_forward_with_a_token_tail_sampled(gpu_lib):
    w = WORKLOADS["skewed_bf16"].with_(T=8191)
    say("[skewed-8191] generating")
    inp = make_inputs(w)
    say(f"[skewed-8191] running T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    d = to_device(inp)
    y = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                            d["down_proj"])
    torch.cuda.synchronize()
    ids = inp["topk_ids"]
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert (counts == 0).sum() >= 3 and (counts[counts > 0] % 256 != 0).any()
    rng = np.random.default_rng(11)
    hot, cold = counts.argmax(), np.where(counts > 0, counts, counts.max() + 1).argmin()
    toks = {0, w.T - 2, w.T - 1}
    toks |= set(np.where((ids == hot).any(1))[0][-3:].tolist())
    toks |= set(np.where((ids == cold).any(1))[0][:3].tolist())
    toks |= set(rng.choice(w.T, 18, replace=False).tolist())
    toks = np.array(sorted(toks), np.int64)
    ref = oracle.forward_tokens(inp["x"], ids, inp["topk_weights"], inp["up_proj"],
                                inp["down_proj"], toks)
    err = max_rel_err(host_f64(y[torch.from_numpy(toks).cuda()]), ref)
    say(f"[skewed-8191] sampled {len(toks)} tokens max_rel_err={err:.3e}")
    assert err <= TOL["bf16"]
    assert torch.isfinite(y.float()).all()
