"""The pipelined forward (tile-granular release) against its bulk twin and the oracle.

The pipelined forward runs GEMM1 and GEMM2 as one persistent launch in which
device counters replace the launch boundary (overlap explainer page, sections
5-6; HyperMegaMoE issue page, tile-level pipelining), then the combine.  It
performs exactly the arithmetic of the bulk forward (the same tiles, the same
accumulation order, the same combine), so its outputs must be bitwise equal to
the bulk twin's, and within the bf16 tolerance of the oracle.  Its tiles are
handed out by tickets, so a single workgroup must also complete it (a test
flag launches one).  The watchdog is exercised from the host: a test flag
drops one release and shortens the watchdog, every wait behind it must time
out and report it (through the status word, and as an error with
MOE_FFN_CHECK_STATUS), and every kernel still ends.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, I, E, K, routing  (all with H % 256 == 0 and I % 128 == 0)
    ("pipe_tiles", 600, 512, 384, 8, 3, "uniform"),
    ("pipe_bm64", 300, 256, 256, 16, 2, "uniform"),
    ("pipe_zipf_empty", 515, 256, 128, 16, 4, "zipf"),
    ("pipe_dups", 129, 256, 128, 4, 3, "replace"),
    ("pipe_one_token", 1, 256, 128, 8, 2, "uniform"),
    ("pipe_k1", 200, 512, 256, 4, 1, "uniform"),
    ("pipe_k32", 40, 256, 128, 64, 32, "uniform"),
]


def fwd(gpu_lib, d, **kw):
    """The pipelined forward unless pipelined=False is passed (the bulk twin)."""
    kw.setdefault("pipelined", True)
    return gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                               d["down_proj"], **kw)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pipelined_equals_bulk_and_oracle(gpu_lib, case):
    name, T, H, I, E, K, routing = case
    w = Workload(name, 400 + CASES.index(case), T=T, H=H, I=I, E=E, K=K, routing=routing,
                 n_empty=3 if routing == "zipf" else 0)
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    say(f"[pipe] case={name} T={T} H={H} I={I} E={E} K={K}")
    y_p, saved_p, ws_p = fwd(gpu_lib, d, save_for_backward=True, return_ws=True)
    y_b, saved_b = fwd(gpu_lib, d, save_for_backward=True, pipelined=False)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws_p) == 0
    assert torch.equal(y_p, y_b)
    # the saved contexts (route arrays and h; their alignment padding is not
    # part of them) must drive the backward to the same bits
    g_p = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                              d["down_proj"], saved_p)
    g_b = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                              d["down_proj"], saved_b)
    torch.cuda.synchronize()
    for a, b in zip(g_p, g_b):
        assert torch.equal(a, b)
    ref = oracle.forward(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"],
                         inp["down_proj"])
    err = max_rel_err(host_f64(y_p), ref)
    say(f"[pipe] case={name} max_rel_err={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("case", [("default_bm64", 300, 256, 256, 16, 2),
                                  ("default_bm128", 600, 512, 384, 8, 3)],
                         ids=["bm64", "bm128"])
def test_default_mode_equals_both_forced_modes(gpu_lib, case):
    # the library's own choice (the pipelined launch on 64-row tiles, the two
    # launches otherwise) gives the same bits as either mode forced
    name, T, H, I, E, K = case
    w = Workload(name, 440 + T, T=T, H=H, I=I, E=E, K=K)
    d = to_device(make_inputs(w))
    prob = gpu_lib.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"])
    rows, family = gpu_lib.fwd_plan(prob)
    assert family == ("pipelined" if rows == 64 else "tiles")
    say(f"[pipe] default vs forced modes case={name} plan=({rows}, {family})")
    y_d = fwd(gpu_lib, d, pipelined=None)
    y_p = fwd(gpu_lib, d, pipelined=True)
    y_b = fwd(gpu_lib, d, pipelined=False)
    torch.cuda.synchronize()
    assert torch.equal(y_d, y_p) and torch.equal(y_d, y_b)


def test_workspace_reuse_sees_fresh_data(gpu_lib):
    # two different batches through one workspace: the second call's consumers
    # must read the second call's tiles, never lines left from the first
    wa = Workload("reuse_a", 420, T=512, H=512, I=256, E=8, K=2)
    wb = Workload("reuse_b", 421, T=512, H=512, I=256, E=8, K=2)
    da, db = to_device(make_inputs(wa)), to_device(make_inputs(wb))
    say("[pipe] workspace reuse")
    _, ws = fwd(gpu_lib, da, return_ws=True)
    for _ in range(3):
        y_a = fwd(gpu_lib, da, ws=ws)
        y_b = fwd(gpu_lib, db, ws=ws)
    ref_a = fwd(gpu_lib, da, pipelined=False)
    ref_b = fwd(gpu_lib, db, pipelined=False)
    torch.cuda.synchronize()
    assert torch.equal(y_a, ref_a) and torch.equal(y_b, ref_b)
    assert gpu_lib.read_status(ws) == 0


def test_int64_ids_match_int32(gpu_lib):
    w = Workload("ids64", 422, T=333, H=256, I=256, E=8, K=3)
    d = to_device(make_inputs(w))
    say("[pipe] int64 ids")
    y32 = fwd(gpu_lib, d)
    d64 = dict(d, topk_ids=d["topk_ids"].to(torch.int64))
    y64 = fwd(gpu_lib, d64)
    torch.cuda.synchronize()
    assert torch.equal(y32, y64)


def test_out_of_range_ids_dropped_like_bulk(gpu_lib):
    w = Workload("badid", 423, T=256, H=256, I=128, E=8, K=2)
    d = to_device(make_inputs(w))
    ids = d["topk_ids"].clone()
    ids[5, 1] = 8
    ids[77, 0] = -1
    d = dict(d, topk_ids=ids)
    say("[pipe] out-of-range ids")
    y_p, ws = fwd(gpu_lib, d, return_ws=True)
    y_b = fwd(gpu_lib, d, pipelined=False)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == gpu_lib.DEV_BAD_ID
    assert torch.equal(y_p, y_b)


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_one_workgroup_completes_the_pipelined_launch(gpu_lib, case):
    name, T, H, I, E, K, routing = case
    w = Workload(name, 400 + CASES.index(case), T=T, H=H, I=I, E=E, K=K, routing=routing,
                 n_empty=3 if routing == "zipf" else 0)
    d = to_device(make_inputs(w))
    say(f"[pipe] one workgroup case={name}")
    y_1, ws = fwd(gpu_lib, d, return_ws=True, flags=gpu_lib.TEST_ONE_WORKGROUP)
    y_b = fwd(gpu_lib, d, pipelined=False)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    assert torch.equal(y_1, y_b)


def test_watchdog_reports_a_dropped_release(gpu_lib):
    w = Workload("drop", 424, T=256, H=256, I=256, E=4, K=2)
    d = to_device(make_inputs(w))
    say("[pipe] dropped release -> watchdog")
    _, ws = fwd(gpu_lib, d, return_ws=True, flags=gpu_lib.TEST_DROP_RELEASE)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) & gpu_lib.DEV_TIMEOUT
    # with MOE_FFN_CHECK_STATUS the call itself fails with MOE_FFN_ERR_TIMEOUT
    with pytest.raises(gpu_lib.MoEFFNError) as ei:
        fwd(gpu_lib, d, flags=gpu_lib.TEST_DROP_RELEASE | gpu_lib.CHECK_STATUS)
    assert ei.value.status == 10
    # the next call on the same workspace starts clean and is exact again
    y = fwd(gpu_lib, d, ws=ws)
    y_b = fwd(gpu_lib, d, pipelined=False)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    assert torch.equal(y, y_b)


@pytest.mark.parametrize("name", ["prefill_bf16", "skewed_bf16", "decode_bf16", "fwdbwd_bf16"])
def test_pipelined_equals_bulk_full_size(gpu_lib, name):
    w = WORKLOADS[name]
    say(f"[pipe-full] generating {name}")
    d = to_device(make_inputs(w, with_dy=False))
    say(f"[pipe-full] running {name}")
    y_p, ws = fwd(gpu_lib, d, return_ws=True)
    y_b = fwd(gpu_lib, d, pipelined=False)
    torch.cuda.synchronize()
    assert gpu_lib.read_status(ws) == 0
    assert torch.equal(y_p, y_b)
    assert torch.isfinite(y_p.float()).all()
