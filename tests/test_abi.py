"""The C-ABI library loads, exports what include/moe_ffn.h declares, and rejects
bad arguments on the host before anything is launched (no GPU needed).

Shapes, dtypes, alignment and buffer sizes are checked at the boundary before
any kernel runs (HyperMegaMoE issue page, section 4.2 "numeric and boundary
constraints"; section 5.3: the host computes and checks the workspace size).
"""

import ctypes

import pytest

import mixture_experts_ffn_amd as m

FAKE = 1 << 40  # an aligned, never-dereferenced address: every call below fails first


@pytest.fixture(scope="module")
def lib():
    return m.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = m.exported_symbols()
    assert "moe_ffn_fwd" in names and "moe_ffn_route" in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version(lib):
    assert lib.moe_ffn_version().decode().count(".") == 2


def prob(**kw):
    base = dict(T=64, H=256, I=128, E=8, K=2, dtype=m.BF16, ids_dtype=m.I32)
    base.update(kw)
    return m.Problem(base["T"], base["H"], base["I"], base["E"], base["K"], base["dtype"],
                     base["ids_dtype"])


@pytest.mark.parametrize("bad,code", [
    (dict(K=0), 2), (dict(K=33), 2), (dict(E=0), 2), (dict(E=1025), 2), (dict(H=12), 2),
    (dict(I=4), 2), (dict(T=-1), 2), (dict(T=1 << 28, K=8), 2), (dict(dtype=7), 3),
    (dict(ids_dtype=m.F32), 3),
])
def test_workspace_query_rejects_bad_problems(bad, code):
    with pytest.raises(m.MoEFFNError) as ei:
        m.fwd_workspace_size(prob(**bad))
    assert ei.value.status == code


@pytest.mark.parametrize("shape,plan", [
    # (T, H, I, E, K): decode, prefill, skewed shapes; rows per expert 32, 384, 2048
    ((128, 7168, 2048, 32, 8), (64, "pipelined")),
    ((4096, 2048, 1408, 64, 6), (128, "tiles_big_gemm2")),
    ((8192, 7168, 2048, 32, 8), (256, "big_tiles")),
    # 225 rows per expert: both GEMMs on 128-row tiles
    ((600, 512, 384, 8, 3), (128, "tiles")),
    # ragged H: the engine
    ((600, 264, 256, 8, 2), (128, "engine")),
])
def test_forward_plan_picks_the_tile_height_from_rows_per_expert(shape, plan):
    T, H, I, E, K = shape
    p = prob(T=T, H=H, I=I, E=E, K=K)
    assert m.fwd_plan(p) == plan
    # the pipelined launch keeps the tile height of the two-launch forward for
    # 64 and 128-row tiles and never takes the 256 x 256 kernel; the library
    # picks it by default on 64-row tiles only
    rows, fam = m.fwd_plan(p, m.PIPELINE)
    bulk = m.fwd_plan(p, m.BULK)
    if plan[1] in ("tiles", "pipelined", "tiles_big_gemm2"):
        assert (rows, fam) == (plan[0], "pipelined")
        assert bulk == (plan[0], "tiles" if plan[1] == "pipelined" else plan[1])
    elif plan[1] == "big_tiles":
        assert fam == "pipelined" and rows in (128, 256)
        assert bulk == plan


def test_workspace_size_grows_with_tokens():
    small, saved_small = m.fwd_workspace_size(prob(T=64))
    big, saved_big = m.fwd_workspace_size(prob(T=4096))
    assert big > small > 0 and saved_big > saved_small > 0
    # act [TK, I] and o [TK, H] in bf16 dominate
    assert big >= 4096 * 2 * (128 + 256) * 2
    # saved holds h [TK, 2I]
    assert saved_big >= 4096 * 2 * 256 * 2


def _fwd(lib, p, x=FAKE, ids=FAKE, g=FAKE, w1=FAKE, w2=FAKE, y=FAKE, saved=None, ws=FAKE,
         ws_bytes=1 << 40, flags=0):
    vp = lambda a: None if a is None else ctypes.c_void_p(a)
    return lib.moe_ffn_fwd(ctypes.byref(p), vp(x), vp(ids), vp(g), vp(w1), vp(w2), vp(y),
                           vp(saved), vp(ws), ws_bytes, flags, None)


def test_fwd_rejects_pipeline_and_bulk_together(lib):
    assert _fwd(lib, prob(), flags=m.PIPELINE | m.BULK) == 2
    assert b"exclude" in lib.moe_ffn_last_error()


def test_fwd_rejects_null_and_misaligned_pointers_before_launch(lib):
    p = prob()
    assert _fwd(lib, p, x=None) == 1
    assert _fwd(lib, p, w2=None) == 1
    assert _fwd(lib, p, ws=None) == 1
    assert _fwd(lib, p, y=FAKE + 2) == 4
    assert _fwd(lib, p, ids=FAKE + 2) == 4
    assert _fwd(lib, p, saved=FAKE + 8) == 4
    assert _fwd(lib, prob(ids_dtype=m.I64), ids=FAKE + 4) == 4
    assert b"NULL" in lib.moe_ffn_last_error() or b"aligned" in lib.moe_ffn_last_error()


def test_fwd_rejects_small_workspace(lib):
    p = prob()
    need, _ = m.fwd_workspace_size(p)
    assert _fwd(lib, p, ws_bytes=need - 1) == 5
    assert b"workspace" in lib.moe_ffn_last_error()


def test_fwd_with_zero_tokens_is_a_no_op(lib):
    assert _fwd(lib, prob(T=0), x=None, ids=None, g=None, w1=None, w2=None, y=None,
                ws=None, ws_bytes=0) == 0


def test_status_strings(lib):
    for code in range(10):
        assert lib.moe_ffn_status_string(code)
    assert lib.moe_ffn_status_string(99) == b"unknown status"


def test_python_layer_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    ids = torch.zeros(4, 2, dtype=torch.int32)
    g = torch.zeros(4, 2)
    w1 = torch.zeros(2, 16, 16, dtype=torch.bfloat16)
    w2 = torch.zeros(2, 8, 16, dtype=torch.bfloat16)
    with pytest.raises(m.MoEFFNError):
        m.moe_ffn_fwd(x, ids, g, w1, w2)
