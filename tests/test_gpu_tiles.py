"""The forward's persistent tile walk at two grid sizes, against the oracle.

The fast-path forward runs persistent workgroups (8 waves per CU), each walking a strided
share of its XCD's tiles (and, in the pipelined launch, waiting on the
releases of the tiles it reads).  Every tile is computed whole by one
workgroup, so the output must not depend on how many workgroups walk the
tiles: these tests run the kernels as 16 workgroups (MOE_FFN_TEST_SMALL_GRID,
many tiles per workgroup and many waits) and at the default grid, and require
bitwise equal outputs, equality with the pipelined launch, and the oracle's
tolerance (max|err| / max|ref| <= 1e-2 for bf16).
"""

import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, I, E, K, Is, routing  (the tile height follows from the rows per expert)
    ("tiles_bm128", 652, 512, 256, 8, 3, 0, "uniform"),
    ("tiles_bm128_zipf_empty", 315, 512, 256, 16, 4, 0, "zipf"),
    ("tiles_bm64", 207, 1024, 512, 16, 4, 0, "uniform"),
    ("tiles_bm256", 2051, 512, 512, 2, 2, 0, "uniform"),
    ("tiles_shared", 600, 512, 256, 8, 3, 512, "uniform"),
    # 257-512 rows per expert: GEMM1 on 128-row tiles, GEMM2 on 256-row tiles
    ("tiles_big_gemm2", 1000, 512, 256, 8, 3, 0, "uniform"),
    ("tiles_big_gemm2_zipf_empty", 1400, 512, 256, 8, 2, 0, "zipf"),
    ("tiles_big_gemm2_shared", 700, 512, 256, 8, 4, 512, "uniform"),
]


def workload(case):
    name, T, H, I, E, K, Is, routing = case
    return Workload(name, 700 + CASES.index(case), T=T, H=H, I=I, E=E, K=K, Is=Is,
                    routing=routing, n_empty=3 if routing == "zipf" else 0)


def fwd(gpu_lib, d, flags=0, **kw):
    sh = ({"shared_up_proj_weight": d["shared_up"], "shared_down_proj_weight": d["shared_down"]}
          if "shared_up" in d else {})
    return gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], flags=flags, **sh, **kw)


def reference(inp):
    if "shared_up" in inp:
        return oracle.forward_shared(inp["x"], inp["topk_ids"], inp["topk_weights"],
                                     inp["up_proj"], inp["down_proj"], inp["shared_up"],
                                     inp["shared_down"])
    return oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                          inp["down_proj"])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grid_size_does_not_change_the_result(gpu_lib, case):
    inp = make_inputs(workload(case))
    d = to_device(inp)
    small = gpu_lib.TEST_SMALL_GRID
    say(f"[tiles] case={case[0]} 16 workgroups and the default grid")
    y_small = fwd(gpu_lib, d, small)
    y_small2 = fwd(gpu_lib, d, small)
    y_default = fwd(gpu_lib, d)
    torch.cuda.synchronize()
    err = max_rel_err(host_f64(y_small), reference(inp))
    say(f"[tiles] case={case[0]} max_rel_err={err:.3e}")
    assert err <= TOL["bf16"]
    assert torch.equal(y_small, y_small2)
    assert torch.equal(y_small, y_default)
    if not case[6]:  # the pipelined launch serves routed experts only
        say(f"[tiles] case={case[0]} pipelined, 16 workgroups")
        y_pipe = fwd(gpu_lib, d, small, pipelined=True)
        torch.cuda.synchronize()
        assert torch.equal(y_pipe, y_small)


# one case per tile height: the GEMM1 that saves h is its own kernel per height
SAVED_CASES = [CASES[0], CASES[2], CASES[3], CASES[5]]


@pytest.mark.parametrize("case", SAVED_CASES, ids=[c[0] for c in SAVED_CASES])
def test_small_grid_saved_context_drives_the_backward(gpu_lib, case):
    inp = make_inputs(workload(case), with_dy=True)
    d = to_device(inp)
    say(f"[tiles] case={case[0]} backward from a 16-workgroup forward")
    y_inf = fwd(gpu_lib, d)
    y_saved, saved = fwd(gpu_lib, d, gpu_lib.TEST_SMALL_GRID, save_for_backward=True)
    grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], saved)
    torch.cuda.synchronize()
    # saving h changes nothing in the forward's arithmetic
    assert torch.equal(y_saved, y_inf)
    ref = oracle.backward(inp["dy"], inp["x"], inp["topk_ids"], inp["topk_weights"],
                          inp["up_proj"], inp["down_proj"])
    for n, g, r in zip(("dx", "d_up", "d_down", "d_topk"), grads, ref):
        e = max_rel_err(host_f64(g), r)
        say(f"[tiles] {n} max_rel_err={e:.3e}")
        assert e <= TOL["bf16"], (n, e)


def test_full_size_forward_is_the_same_on_every_call(gpu_lib):
    # the ~2400 GEMM1 and ~1800 GEMM2 tiles of the prefill workload, four bulk
    # calls and a pipelined one: the output must not change
    from synth import WORKLOADS
    w = WORKLOADS["prefill_bf16"]
    say("[tiles-full] generating prefill_bf16")
    d = to_device(make_inputs(w))
    ys = [fwd(gpu_lib, d) for _ in range(4)]
    ys.append(fwd(gpu_lib, d, pipelined=True))
    torch.cuda.synchronize()
    for i, y in enumerate(ys[1:], 1):
        say(f"[tiles-full] call {i} equal={torch.equal(y, ys[0])}")
        assert torch.equal(y, ys[0])


def test_many_experts_three_launch_routing_with_256_row_gemm2(gpu_lib):
    # More than 910 experts: routing runs as three launches (histogram, scan,
    # scatter), and its scan also builds the 256-row M-tile tables; about 261
    # rows per expert put GEMM2 alone on 256 x 256 tiles.  Checked bit for bit
    # against the pipelined launch (both GEMMs on 128-row tiles, tables of the
    # one-table routing) and on sampled tokens against the oracle.
    import numpy as np

    w = Workload("many_experts_big_gemm2", 760, T=30000, H=256, I=128, E=920, K=8)
    say("[tiles-many] generating T=30000 H=256 I=128 E=920 K=8")
    inp = make_inputs(w)
    d = to_device(inp)
    prob = gpu_lib.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"])
    assert gpu_lib.fwd_plan(prob) == (128, "tiles_big_gemm2")
    say("[tiles-many] default and pipelined forwards")
    y = fwd(gpu_lib, d)
    y_pipe = fwd(gpu_lib, d, pipelined=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y_pipe)
    rng = np.random.default_rng(5)
    toks = np.array(sorted({0, w.T - 1} | set(rng.choice(w.T, 30, replace=False).tolist())))
    ref = oracle.forward_tokens(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                                inp["down_proj"], toks)
    err = max_rel_err(host_f64(y[torch.from_numpy(toks).cuda()]), ref)
    say(f"[tiles-many] sampled {len(toks)} tokens max_rel_err={err:.3e}")
    assert err <= TOL["bf16"]
