"""moe_ffn_fwd_noalloc, the forward that allocates nothing (its workspace is
the library's per-GPU scratch), against moe_ffn_fwd with a caller workspace.

Both run the same kernels on the same inputs, so the outputs must agree bit
for bit.  Each pair of calls runs a problem and then a smaller one, so the
second call finds the first call's contents in the scratch.  The calls go
through the C ABI directly (ctypes), not through the Python wrapper.
"""

import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_ffn_amd as m
from gpu_util import say, to_device
from synth import Workload, make_inputs, workload

pytestmark = pytest.mark.gpu

# (name, T, H, I, E, K, dtype, routing): a bf16 shape on 64-row tiles, one on
# the 256 x 256 tile kernel (more than 512 rows per expert), one on 128-row
# tiles, one with GEMM2 alone on 256-row tiles (257-512 rows per expert), a
# ragged bf16 shape (the engine), fp32 (the generic kernels)
PAIRS = [
    ("bf16_bm64", (200, 1024, 512, 16, 4, "bf16", "uniform"), 37),
    ("bf16_big_tiles", (1024, 512, 256, 4, 4, "bf16", "uniform"), 300),
    ("bf16_bm128", (600, 512, 384, 8, 3, "bf16", "zipf"), 129),
    ("bf16_big_gemm2", (1000, 512, 256, 8, 3, "bf16", "uniform"), 700),
    ("bf16_ragged", (333, 264, 200, 6, 2, "bf16", "uniform"), 65),
    ("f32", (256, 256, 512, 8, 2, "f32", "uniform"), 31),
]


def _call_noalloc(lib, d, y, flags=0):
    prob = m.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"])
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.moe_ffn_fwd_noalloc(ctypes.byref(prob), vp(d["x"]), vp(d["topk_ids"]),
                                   vp(d["topk_weights"]), vp(d["up_proj"]), vp(d["down_proj"]),
                                   vp(y), flags, stream)


def _check_pair(gpu_lib, name, shape, t_small, seed, flags=0):
    T, H, I, E, K, dtype, routing = shape
    lib = gpu_lib.load_library()
    for t in (T, t_small):
        w = Workload(name, seed, T=t, H=H, I=I, E=E, K=K, dtype=dtype, routing=routing,
                     n_empty=3 if routing == "zipf" else 0)
        d = to_device(make_inputs(w))
        say(f"[noalloc] case={name} T={t} H={H} I={I} E={E} K={K} {dtype} flags={flags}")
        ws_bytes, _ = gpu_lib.fwd_workspace_size(
            gpu_lib.make_problem(d["x"], d["topk_ids"], d["up_proj"], d["down_proj"]), flags)
        assert ws_bytes <= gpu_lib.NOALLOC_WS_BYTES
        y_ref = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                    d["down_proj"], flags=flags)
        y = torch.full_like(y_ref, float("nan"))
        rc = _call_noalloc(lib, d, y, flags)
        assert rc == 0, lib.moe_ffn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), name


@pytest.mark.parametrize("case", PAIRS, ids=[c[0] for c in PAIRS])
def test_noalloc_equals_fwd_on_two_calls(gpu_lib, case):
    name, shape, t_small = case
    _check_pair(gpu_lib, name, shape, t_small, 700 + PAIRS.index(case))


def test_noalloc_pipelined_equals_fwd(gpu_lib):
    _check_pair(gpu_lib, "bf16_pipelined", (300, 512, 256, 8, 2, "bf16", "uniform"), 41, 720,
                flags=m.PIPELINE)


def test_noalloc_decode_workload_full_size(gpu_lib):
    """The decode workload (the serving-loop caller) at full size."""
    w = workload("decode_bf16")
    d = to_device(make_inputs(w))
    say(f"[noalloc] decode T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    y_ref = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"])
    lib = gpu_lib.load_library()
    y = torch.full_like(y_ref, float("nan"))
    assert _call_noalloc(lib, d, y) == 0, lib.moe_ffn_last_error()
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)


def test_noalloc_rejects_before_launch(gpu_lib):
    lib = gpu_lib.load_library()
    # a workspace beyond the scratch: rejected, y untouched
    w = Workload("noalloc_big", 730, T=4096, H=2048, I=1408, E=64, K=6, dtype="bf16")
    prob = m.Problem(w.T, w.H, w.I, w.E, w.K, m.BF16, m.I32)
    need, _ = m.fwd_workspace_size(prob)
    assert need > m.NOALLOC_WS_BYTES
    x = torch.zeros(8, 16, dtype=torch.bfloat16, device="cuda")  # never read
    y = torch.full((8, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    fake = ctypes.c_void_p(x.data_ptr())
    rc = lib.moe_ffn_fwd_noalloc(ctypes.byref(prob), fake, fake, fake, fake, fake,
                                 ctypes.c_void_p(y.data_ptr()), 0, None)
    assert rc == 5 and b"scratch" in lib.moe_ffn_last_error()
    # MOE_FFN_CHECK_IDS copies to the host: rejected
    small = m.Problem(8, 256, 128, 4, 2, m.BF16, m.I32)
    rc = lib.moe_ffn_fwd_noalloc(ctypes.byref(small), fake, fake, fake, fake, fake,
                                 ctypes.c_void_p(y.data_ptr()), m.CHECK_IDS, None)
    assert rc == 2 and b"CHECK_IDS" in lib.moe_ffn_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
