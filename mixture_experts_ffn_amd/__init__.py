"""MI355X (gfx950) MoE expert-FFN layer: Python binding of ``libmoe_ffn.so``.

The binding only marshals arguments: every step of the layer (routing,
gathered up_proj GEMM with SwiGLU, down_proj GEMM, combine, and the backward)
runs in the HIP kernels of the library.  PyTorch provides device memory and
the current stream.  There is no CPU or eager fallback: if the library is not
built, or the tensors are not on a GPU, the calls raise.

Public API (names follow the C ABI of ``include/moe_ffn.h``):

* ``moe_ffn_fwd(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
  save_for_backward=False, check_ids=False)`` -> ``y`` (and the saved context)
* ``moe_ffn_route(topk_ids, E)`` -> counts, offsets, sorted_slot, slot_pos
* ``moe_ffn(...)`` autograd-aware layer (forward + backward through the library)
"""

from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

__all__ = [
    "MoEFFNError",
    "load_library",
    "library_path",
    "exported_symbols",
    "Problem",
    "StageEvents",
    "fwd_workspace_size",
    "route_workspace_size",
    "moe_ffn_fwd",
    "moe_ffn_fwd_noalloc",
    "NOALLOC_WS_BYTES",
    "fwd_stages",
    "fwd_plan",
    "moe_ffn_route",
    "read_status",
    "STAGES",
    "BWD_STAGES",
    "bwd_workspace_size",
    "moe_ffn_bwd_d",
    "moe_ffn_bwd_w",
    "moe_ffn_bwd",
    "moe_ffn",
    "MoEFFNFunction",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmoe_ffn.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe_ffn.h")
_lock = threading.Lock()
_lib = None

F32, BF16, I32, I64 = 0, 1, 2, 3
CHECK_IDS = 0x1
PIPELINE = 0x2
BULK = 0x10
CHECK_STATUS = 0x8
TEST_ONE_WORKGROUP = 0x400
TEST_DROP_RELEASE = 0x100
TEST_SMALL_GRID = 0x200
CHECK_SAVED = 0x4
DEV_BAD_ID, DEV_TIMEOUT, DEV_BAD_SAVED, DEV_BAD_WS = 0x1, 0x2, 0x4, 0x8
STAGES = ("route", "gemm1", "gemm2", "combine", "pipeline")
BWD_STAGES = ("act_grad", "input_grad", "dx_combine", "w2_grad", "w1_grad")

ERR_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
             5: "ERR_WORKSPACE", 6: "ERR_EXPERT_ID", 7: "ERR_SAVED", 8: "ERR_HIP",
             9: "ERR_DEVICE", 10: "ERR_TIMEOUT"}


class MoEFFNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{ERR_NAMES.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int64), ("K", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("ids_dtype", ctypes.c_int32), ("Is", ctypes.c_int64)]


class SharedWeights(ctypes.Structure):
    _fields_ = [("up_proj_weight", ctypes.c_void_p), ("down_proj_weight", ctypes.c_void_p)]


class SharedGrads(ctypes.Structure):
    _fields_ = [("d_up_proj_weight", ctypes.c_void_p), ("d_down_proj_weight", ctypes.c_void_p)]


class FwdStageLayout(ctypes.Structure):
    """Byte offsets of the forward's intermediate stages in its workspace."""

    _fields_ = [(n, ctypes.c_size_t) for n in
                ("counts", "offsets", "sorted_slot", "slot_pos", "act", "o")] + \
               [("tile_rows", ctypes.c_int32), ("kernel", ctypes.c_int32)]


KERNELS = {0: "generic", 1: "engine", 2: "tiles", 3: "big_tiles", 4: "pipelined",
           5: "tiles_big_gemm2"}


def fwd_plan(problem: Problem, flags: int = 0):
    """(tile rows, kernel family name) the forward runs for this problem."""
    lay = FwdStageLayout()
    _check(load_library().moe_ffn_fwd_stages(ctypes.byref(problem), flags, ctypes.byref(lay)))
    return lay.tile_rows, KERNELS[lay.kernel]


class StageEvents(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_void_p * 8), ("end", ctypes.c_void_p * 8)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmoe_ffn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m mixture_experts_ffn_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
        pp = ctypes.POINTER(Problem)
        psz = ctypes.POINTER(ctypes.c_size_t)
        sigs = {
            "moe_ffn_fwd_workspace_size": [pp, u32, psz, psz],
            "moe_ffn_fwd": [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
            "moe_ffn_fwd_ex": [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp,
                               ctypes.POINTER(StageEvents)],
            "moe_ffn_route_workspace_size": [pp, psz],
            "moe_ffn_bwd_workspace_size": [pp, u32, psz],
            "moe_ffn_bwd": [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
            "moe_ffn_bwd_ex": [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp,
                               ctypes.POINTER(StageEvents)],
            "moe_ffn_bwd_d": [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
            "moe_ffn_fwd_shared": [pp, vp, vp, vp, vp, vp, ctypes.POINTER(SharedWeights), vp, vp,
                                   vp, sz, u32, vp, ctypes.POINTER(StageEvents)],
            "moe_ffn_bwd_shared": [pp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(SharedWeights), vp,
                                   vp, vp, vp, vp, ctypes.POINTER(SharedGrads), vp, sz, u32, vp,
                                   ctypes.POINTER(StageEvents)],
            "moe_ffn_bwd_w": [pp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
            "moe_ffn_route": [pp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_ffn_fwd_noalloc": [pp, vp, vp, vp, vp, vp, vp, u32, vp],
            "moe_ffn_fwd_stages": [pp, u32, ctypes.POINTER(FwdStageLayout)],
            "moe_ffn_read_status": [vp, vp, ctypes.POINTER(ctypes.c_int32)],
            "moe_ffn_event_create": [ctypes.POINTER(ctypes.c_void_p)],
            "moe_ffn_event_destroy": [vp],
            "moe_ffn_event_elapsed_ms": [vp, vp, ctypes.POINTER(ctypes.c_float)],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = i32
        for name in ("moe_ffn_status_string",):
            getattr(lib, name).argtypes = [i32]
            getattr(lib, name).restype = ctypes.c_char_p
        lib.moe_ffn_last_error.argtypes = []
        lib.moe_ffn_last_error.restype = ctypes.c_char_p
        lib.moe_ffn_version.argtypes = []
        lib.moe_ffn_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def exported_symbols() -> list[str]:
    """Function names declared in include/moe_ffn.h."""
    text = open(_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ffn_\w+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        detail = lib.moe_ffn_last_error().decode() or lib.moe_ffn_status_string(rc).decode()
        raise MoEFFNError(rc, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise MoEFFNError(3, f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ids_code(t: torch.Tensor) -> int:
    if t.dtype == torch.int32:
        return I32
    if t.dtype == torch.int64:
        return I64
    raise MoEFFNError(3, f"topk_ids must be int32 or int64, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MoEFFNError(1, "all tensors must be on the GPU (no CPU fallback exists)")
        if t is not None and not t.is_contiguous():
            raise MoEFFNError(4, "all tensors must be contiguous")


def make_problem(x, topk_ids, up_proj_weight, down_proj_weight) -> Problem:
    if x.dim() != 2 or topk_ids.dim() != 2 or up_proj_weight.dim() != 3 or down_proj_weight.dim() != 3:
        raise MoEFFNError(2, "expected x [T,H], topk_ids [T,K], up [E,H,2I], down [E,I,H]")
    T, H = x.shape
    E, H2, I2 = up_proj_weight.shape
    E2, I, H3 = down_proj_weight.shape
    if topk_ids.shape[0] != T or H2 != H or H3 != H or E2 != E or I2 != 2 * I:
        raise MoEFFNError(2, f"inconsistent shapes x{tuple(x.shape)} ids{tuple(topk_ids.shape)} "
                             f"up{tuple(up_proj_weight.shape)} down{tuple(down_proj_weight.shape)}")
    if up_proj_weight.dtype != x.dtype or down_proj_weight.dtype != x.dtype:
        raise MoEFFNError(3, "x, up_proj_weight and down_proj_weight must share one dtype")
    return Problem(T, H, I, E, topk_ids.shape[1], _dtype_code(x), _ids_code(topk_ids))


def fwd_workspace_size(problem: Problem, flags: int = 0):
    ws, saved = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().moe_ffn_fwd_workspace_size(ctypes.byref(problem), flags,
                                                     ctypes.byref(ws), ctypes.byref(saved)))
    return ws.value, saved.value


def route_workspace_size(problem: Problem) -> int:
    ws = ctypes.c_size_t()
    _check(load_library().moe_ffn_route_workspace_size(ctypes.byref(problem), ctypes.byref(ws)))
    return ws.value


def _shared_problem(prob, x, shared_up_proj_weight, shared_down_proj_weight):
    """Set prob.Is from the shared-expert weights (both or neither)."""
    if shared_up_proj_weight is None and shared_down_proj_weight is None:
        return None
    if shared_up_proj_weight is None or shared_down_proj_weight is None:
        raise MoEFFNError(2, "pass both shared_up_proj_weight and shared_down_proj_weight")
    _require_gpu(shared_up_proj_weight, shared_down_proj_weight)
    Is, H = shared_down_proj_weight.shape
    if shared_up_proj_weight.shape != (H, 2 * Is) or H != x.shape[1]:
        raise MoEFFNError(2, "expected shared_up [H, 2Is] and shared_down [Is, H]")
    if shared_up_proj_weight.dtype != x.dtype or shared_down_proj_weight.dtype != x.dtype:
        raise MoEFFNError(3, "the shared weights must have the dtype of x")
    prob.Is = Is
    return SharedWeights(shared_up_proj_weight.data_ptr(), shared_down_proj_weight.data_ptr())


def _mode_flag(pipelined):
    """MOE_FFN_PIPELINE for True, MOE_FFN_BULK for False, nothing for None."""
    if pipelined is None:
        return 0
    return PIPELINE if pipelined else BULK


def moe_ffn_fwd(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, *,
                save_for_backward: bool = False, check_ids: bool = False, ws=None,
                stage_events: StageEvents | None = None, return_ws: bool = False,
                pipelined: bool | None = None, flags: int = 0, shared_up_proj_weight=None,
                shared_down_proj_weight=None):
    """y [T, H] of the MoE expert-FFN layer (see include/moe_ffn.h).

    With ``save_for_backward`` also returns the saved context (a uint8 device
    tensor) that the backward consumes.  ``ws`` may pass a preallocated
    workspace (uint8 tensor of at least ``fwd_workspace_size`` bytes).
    ``pipelined`` True asks for the one-launch forward with tile-granular
    release (bf16, H % 256 == 0, I % 128 == 0; other shapes ignore it), False
    for the two separate GEMM launches, None (the default) leaves the choice
    to the library;
    ``flags`` passes further MOE_FFN_* bits through.  ``shared_up_proj_weight``
    [H, 2Is] and ``shared_down_proj_weight`` [Is, H] (Is a multiple of I) add the
    shared expert's SwiGLU FFN to y; the saved context then covers it too.
    """
    lib = load_library()
    _require_gpu(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)
    if topk_weights.dtype != torch.float32 or topk_weights.shape != topk_ids.shape:
        raise MoEFFNError(3, "topk_weights must be float32 with the shape of topk_ids")
    prob = make_problem(x, topk_ids, up_proj_weight, down_proj_weight)
    sw = _shared_problem(prob, x, shared_up_proj_weight, shared_down_proj_weight)
    ws_bytes, saved_bytes = fwd_workspace_size(prob)
    dev = x.device
    y = torch.empty_like(x)
    if ws is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif ws.numel() < ws_bytes:
        raise MoEFFNError(5, f"workspace has {ws.numel()} bytes, {ws_bytes} needed")
    saved = torch.empty(saved_bytes, dtype=torch.uint8, device=dev) if save_for_backward else None
    flags |= (CHECK_IDS if check_ids else 0) | _mode_flag(pipelined)
    ev = ctypes.byref(stage_events) if stage_events is not None else None
    with torch.cuda.device(dev):
        if sw is not None:
            rc = lib.moe_ffn_fwd_shared(ctypes.byref(prob), _ptr(x), _ptr(topk_ids),
                                        _ptr(topk_weights), _ptr(up_proj_weight),
                                        _ptr(down_proj_weight), ctypes.byref(sw), _ptr(y),
                                        _ptr(saved), _ptr(ws), ws.numel(), flags, _stream(dev),
                                        ev)
        else:
            rc = lib.moe_ffn_fwd_ex(ctypes.byref(prob), _ptr(x), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(up_proj_weight),
                                    _ptr(down_proj_weight), _ptr(y), _ptr(saved), _ptr(ws),
                                    ws.numel(), flags, _stream(dev), ev)
    _check(rc)
    out = (y,)
    if save_for_backward:
        out += (saved,)
    if return_ws:
        out += (ws,)
    return out[0] if len(out) == 1 else out


def fwd_stages(x, topk_ids, up_proj_weight, down_proj_weight, ws, flags: int = 0):
    """Views of the intermediate stages an inference forward left in ``ws``:
    counts, offsets, sorted_slot, slot_pos (int32) and act [TK, I], o [TK, H]
    in the problem dtype, rows in permuted (expert-major) order."""
    prob = make_problem(x, topk_ids, up_proj_weight, down_proj_weight)
    lay = FwdStageLayout()
    _check(load_library().moe_ffn_fwd_stages(ctypes.byref(prob), flags, ctypes.byref(lay)))
    T, K, E = prob.T, prob.K, prob.E
    I, H = prob.I, prob.H

    def view(off, n, dtype, shape):
        nb = n * torch.empty((), dtype=dtype).element_size()
        return ws[off:off + nb].view(dtype).view(shape)

    return dict(counts=view(lay.counts, E, torch.int32, (E,)),
                offsets=view(lay.offsets, E + 1, torch.int32, (E + 1,)),
                sorted_slot=view(lay.sorted_slot, T * K, torch.int32, (T * K,)),
                slot_pos=view(lay.slot_pos, T * K, torch.int32, (T * K,)),
                act=view(lay.act, T * K * I, x.dtype, (T * K, I)),
                o=view(lay.o, T * K * H, x.dtype, (T * K, H)))


def moe_ffn_fwd_noalloc(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, y, *,
                        pipelined: bool | None = None, flags: int = 0):
    """The inference forward into the caller's ``y`` [T, H] with no workspace:
    the library's own per-GPU scratch (include/moe_ffn.h, moe_ffn_fwd_noalloc)
    serves as the workspace, so nothing is allocated.  Raises MoEFFNError for
    problems whose workspace exceeds NOALLOC_WS_BYTES."""
    lib = load_library()
    _require_gpu(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, y)
    if topk_weights.dtype != torch.float32 or topk_weights.shape != topk_ids.shape:
        raise MoEFFNError(3, "topk_weights must be float32 with the shape of topk_ids")
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise MoEFFNError(2, "y must be a contiguous tensor with the shape and dtype of x")
    prob = make_problem(x, topk_ids, up_proj_weight, down_proj_weight)
    flags |= _mode_flag(pipelined)
    dev = x.device
    with torch.cuda.device(dev):
        rc = lib.moe_ffn_fwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(topk_ids),
                                     _ptr(topk_weights), _ptr(up_proj_weight),
                                     _ptr(down_proj_weight), _ptr(y), flags, _stream(dev))
    _check(rc)
    return y


NOALLOC_WS_BYTES = 64 << 20  # MOE_FFN_NOALLOC_WS_BYTES


def bwd_workspace_size(problem: Problem, flags: int = 0) -> int:
    ws = ctypes.c_size_t()
    _check(load_library().moe_ffn_bwd_workspace_size(ctypes.byref(problem), flags,
                                                     ctypes.byref(ws)))
    return ws.value


def moe_ffn_bwd(dy, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, saved, *,
                ws=None, stage_events: StageEvents | None = None, check_saved: bool = False,
                return_ws: bool = False, shared_up_proj_weight=None,
                shared_down_proj_weight=None):
    """Gradients (dx, d_up_proj_weight, d_down_proj_weight, d_topk_weights) of the layer.

    With the shared expert's weights (as given to the forward) it also returns
    (d_shared_up_proj_weight, d_shared_down_proj_weight).

    `saved` is the context returned by ``moe_ffn_fwd(..., save_for_backward=True)`` for the
    same inputs.  Outputs are freshly allocated and overwritten (never accumulated).
    ``check_saved`` verifies on the host (synchronously) that `saved` belongs to this
    problem; otherwise the check runs on the device and a mismatch yields zeros and the
    DEV_BAD_SAVED status bit (``read_status`` of the workspace, see ``return_ws``).
    """
    lib = load_library()
    _require_gpu(dy, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, saved)
    prob = make_problem(x, topk_ids, up_proj_weight, down_proj_weight)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise MoEFFNError(2, "dy must have the shape and dtype of x")
    sw = _shared_problem(prob, x, shared_up_proj_weight, shared_down_proj_weight)
    ws_bytes = bwd_workspace_size(prob)
    dev = x.device
    dx = torch.empty_like(x)
    d_up = torch.empty_like(up_proj_weight)
    d_down = torch.empty_like(down_proj_weight)
    d_topk = torch.empty(topk_ids.shape, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ev = ctypes.byref(stage_events) if stage_events is not None else None
    flags = CHECK_SAVED if check_saved else 0
    with torch.cuda.device(dev):
        if sw is not None:
            d_sup = torch.empty_like(shared_up_proj_weight)
            d_sdown = torch.empty_like(shared_down_proj_weight)
            sg = SharedGrads(d_sup.data_ptr(), d_sdown.data_ptr())
            rc = lib.moe_ffn_bwd_shared(ctypes.byref(prob), _ptr(dy), _ptr(x), _ptr(topk_ids),
                                        _ptr(topk_weights), _ptr(up_proj_weight),
                                        _ptr(down_proj_weight), ctypes.byref(sw), _ptr(saved),
                                        _ptr(dx), _ptr(d_up), _ptr(d_down), _ptr(d_topk),
                                        ctypes.byref(sg), _ptr(ws), ws.numel(), flags,
                                        _stream(dev), ev)
        else:
            rc = lib.moe_ffn_bwd_ex(ctypes.byref(prob), _ptr(dy), _ptr(x), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(up_proj_weight),
                                    _ptr(down_proj_weight), _ptr(saved), _ptr(dx), _ptr(d_up),
                                    _ptr(d_down), _ptr(d_topk), _ptr(ws), ws.numel(), flags,
                                    _stream(dev), ev)
    _check(rc)
    if sw is not None:
        return (dx, d_up, d_down, d_topk, d_sup, d_sdown) + ((ws,) if return_ws else ())
    if return_ws:
        return dx, d_up, d_down, d_topk, ws
    return dx, d_up, d_down, d_topk


def moe_ffn_bwd_d(dy, topk_ids, topk_weights, up_proj_weight, down_proj_weight, saved, *,
                  ws=None, check_saved: bool = False):
    """Data half of the backward: (dx, d_topk_weights, ws).

    `ws` then holds the intermediate gradients that ``moe_ffn_bwd_w`` reads; keep it
    untouched until that call has been issued on the same stream.
    """
    lib = load_library()
    _require_gpu(dy, topk_ids, topk_weights, up_proj_weight, down_proj_weight, saved)
    prob = make_problem(dy, topk_ids, up_proj_weight, down_proj_weight)
    ws_bytes = bwd_workspace_size(prob)
    dev = dy.device
    dx = torch.empty_like(dy)
    d_topk = torch.empty(topk_ids.shape, dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    flags = CHECK_SAVED if check_saved else 0
    with torch.cuda.device(dev):
        rc = lib.moe_ffn_bwd_d(ctypes.byref(prob), _ptr(dy), _ptr(topk_weights),
                               _ptr(up_proj_weight), _ptr(down_proj_weight), _ptr(saved), _ptr(dx),
                               _ptr(d_topk), _ptr(ws), ws.numel(), flags, _stream(dev))
    _check(rc)
    return dx, d_topk, ws


def moe_ffn_bwd_w(dy, x, topk_ids, up_proj_weight, down_proj_weight, saved, ws, *,
                  check_saved: bool = False):
    """Weight half of the backward: (d_up_proj_weight, d_down_proj_weight).

    `ws` must be the workspace of the ``moe_ffn_bwd_d`` call for the same `saved`
    context; otherwise the gradients are zeros and ``read_status(ws)`` has DEV_BAD_WS
    (with ``check_saved`` the call raises instead).  topk_ids and the weights only
    describe the problem's shape here.
    """
    lib = load_library()
    _require_gpu(dy, x, topk_ids, saved, ws)
    prob = make_problem(x, topk_ids, up_proj_weight, down_proj_weight)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise MoEFFNError(2, "dy must have the shape and dtype of x")
    dev = x.device
    d_up = torch.empty_like(up_proj_weight)
    d_down = torch.empty_like(down_proj_weight)
    flags = CHECK_SAVED if check_saved else 0
    with torch.cuda.device(dev):
        rc = lib.moe_ffn_bwd_w(ctypes.byref(prob), _ptr(dy), _ptr(x), _ptr(saved), _ptr(d_up),
                               _ptr(d_down), _ptr(ws), ws.numel(), flags, _stream(dev))
    _check(rc)
    return d_up, d_down


class MoEFFNFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves the library's context (route arrays and the
    pre-activation), backward returns one gradient per input (None for topk_ids)."""

    @staticmethod
    def forward(ctx, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight):
        y, saved = moe_ffn_fwd(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
                               save_for_backward=True)
        ctx.save_for_backward(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
                              saved)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, topk_ids, topk_weights, up, down, saved = ctx.saved_tensors
        dx, d_up, d_down, d_topk = moe_ffn_bwd(dy.contiguous(), x, topk_ids, topk_weights, up,
                                               down, saved)
        return dx, None, d_topk, d_up, d_down


def moe_ffn(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight):
    """y = MoE expert-FFN layer; differentiable in x, topk_weights and both weights."""
    return MoEFFNFunction.apply(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)


def moe_ffn_route(topk_ids: torch.Tensor, E: int, H: int = 8, I: int = 8):
    """Routing alone: (counts [E], offsets [E+1], sorted_slot [TK], slot_pos [TK], ws)."""
    lib = load_library()
    _require_gpu(topk_ids)
    T, K = topk_ids.shape
    prob = Problem(T, H, I, E, K, BF16, _ids_code(topk_ids))
    ws_bytes = route_workspace_size(prob)
    dev = topk_ids.device
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slot = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
    slot_pos = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        rc = lib.moe_ffn_route(ctypes.byref(prob), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                               _ptr(sorted_slot), _ptr(slot_pos), _ptr(ws), ws_bytes,
                               _stream(dev))
    _check(rc)
    return counts, offsets, sorted_slot[:T * K], slot_pos[:T * K], ws


def read_status(ws: torch.Tensor) -> int:
    """Device status word of the last forward/route on `ws` (DEV_BAD_ID | DEV_TIMEOUT bits)."""
    lib = load_library()
    st = ctypes.c_int32()
    with torch.cuda.device(ws.device):
        _check(lib.moe_ffn_read_status(_ptr(ws), _stream(ws.device), ctypes.byref(st)))
    return st.value


class EventPool:
    """hipEvents (through the library's helpers) for the per-stage timing hook."""

    def __init__(self, n_sets: int, n_stages: int = 5):
        self.lib = load_library()
        self.sets = []
        for _ in range(n_sets):
            ev = StageEvents()
            for s in range(n_stages):
                for arr in (ev.begin, ev.end):
                    h = ctypes.c_void_p()
                    _check(self.lib.moe_ffn_event_create(ctypes.byref(h)))
                    arr[s] = h
            self.sets.append(ev)
        self.n_stages = n_stages

    def elapsed_ms(self, i: int, stage: int) -> float:
        ms = ctypes.c_float()
        ev = self.sets[i]
        _check(self.lib.moe_ffn_event_elapsed_ms(ev.begin[stage], ev.end[stage], ctypes.byref(ms)))
        return ms.value

    def close(self):
        for ev in self.sets:
            for s in range(self.n_stages):
                for arr in (ev.begin, ev.end):
                    if arr[s]:
                        self.lib.moe_ffn_event_destroy(arr[s])
                        arr[s] = None
        self.sets = []
