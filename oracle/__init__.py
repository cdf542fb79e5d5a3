"""CPU oracle of the MoE expert-FFN layer (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never touches it, and it shares no code with them.

The arithmetic lives in ``moe_oracle.c`` (plain C, double accumulation,
OpenMP over independent rows).  This module compiles it with gcc on first use
(or when ``build()`` is called) and wraps it with ctypes.  Inputs are numpy
arrays: fp32, or bf16 carried as uint16 bit patterns; ``topk_ids`` int32 or
int64; ``topk_weights`` fp32.  Outputs are float64 (route arrays int32).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1
I32, I64 = 0, 1
ERRORS = {1: "expert id out of range", 2: "bad argument", 3: "out of memory",
          4: "combine-protocol invariant failed"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into libmoe_oracle.so next to it."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.moe_oracle_route.argtypes = [i64, i64, i64, vp, i32, vp, vp, vp, vp]
    lib.moe_oracle_fwd.argtypes = [i64] * 5 + [i32, vp, vp, i32, vp, vp, vp, vp] + [vp] * 6
    lib.moe_oracle_fwd_tokens.argtypes = [i64] * 5 + [i32, vp, vp, i32, vp, vp, vp, vp, i64, vp]
    lib.moe_oracle_bwd.argtypes = [i64] * 5 + [i32, vp, vp, vp, i32, vp, vp, vp] + [vp] * 4
    lib.moe_oracle_bwd_sampled.argtypes = ([i64] * 5 + [i32, vp, vp, vp, i32, vp, vp, vp, vp, i64,
                                                        vp, vp, vp, i64, vp, vp, i64, vp])
    for fn in ("moe_oracle_route", "moe_oracle_fwd", "moe_oracle_fwd_tokens", "moe_oracle_bwd",
               "moe_oracle_bwd_sampled", "moe_oracle_max_threads"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


_variant = threading.local()


def use_library(path: str | None):
    """Route this thread's oracle calls to another build of moe_oracle.c (or back, with None).

    Only the mutation tests use this: they compile a copy of the source with a
    planted mistake and check that the pins reject it.
    """
    _variant.lib = None if path is None else _bind(path)


def _load():
    global _lib
    v = getattr(_variant, "lib", None)
    if v is not None:
        return v
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().moe_oracle_max_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes fp32 or bf16-as-uint16, got {a.dtype}")


def _idt(a: np.ndarray) -> int:
    if a.dtype == np.int32:
        return I32
    if a.dtype == np.int64:
        return I64
    raise TypeError(f"topk_ids must be int32 or int64, got {a.dtype}")


def _check(rc: int):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, f"oracle error {rc}"))


def _shapes(x, ids, up, down):
    T, H = x.shape
    K = ids.shape[1]
    E, H2, I2 = up.shape
    I = down.shape[1]
    if H2 != H or I2 != 2 * I or down.shape != (E, I, H) or ids.shape[0] != T:
        raise ValueError("inconsistent shapes")
    return T, H, I, E, K


def route(topk_ids: np.ndarray, E: int):
    """Counting sort of the T*K slots, stable in slot index s = t*K + k.

    Returns counts [E], offsets [E+1], sorted_slot [TK], slot_pos [TK] (int32).
    """
    ids = np.ascontiguousarray(topk_ids)
    T, K = ids.shape
    TK = T * K
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_slot = np.zeros(max(TK, 1), np.int32)
    slot_pos = np.zeros(max(TK, 1), np.int32)
    _check(_load().moe_oracle_route(T, K, E, _p(ids), _idt(ids), _p(counts), _p(offsets),
                                    _p(sorted_slot), _p(slot_pos)))
    return counts, offsets, sorted_slot[:TK], slot_pos[:TK]


def forward(x, topk_ids, topk_weights, up_proj, down_proj, *, intermediates=False):
    """y [T,H] float64 (plus route arrays, act and o in permuted order if asked)."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(topk_ids)
    g = np.ascontiguousarray(topk_weights, dtype=np.float32)
    up = np.ascontiguousarray(up_proj)
    down = np.ascontiguousarray(down_proj)
    T, H, I, E, K = _shapes(x, ids, up, down)
    dt = _dt(x)
    assert _dt(up) == dt and _dt(down) == dt
    TK = T * K
    y = np.zeros((T, H), np.float64)
    if intermediates:
        counts = np.zeros(E, np.int32)
        offsets = np.zeros(E + 1, np.int32)
        ss = np.zeros(max(TK, 1), np.int32)
        sp = np.zeros(max(TK, 1), np.int32)
        act = np.zeros((max(TK, 1), I), np.float64)
        o = np.zeros((max(TK, 1), H), np.float64)
    else:
        counts = offsets = ss = sp = act = o = None
    _check(_load().moe_oracle_fwd(T, H, I, E, K, dt, _p(x), _p(ids), _idt(ids), _p(g), _p(up),
                                  _p(down), _p(y), _p(counts), _p(offsets), _p(ss), _p(sp),
                                  _p(act), _p(o)))
    if not intermediates:
        return y
    return y, dict(counts=counts, offsets=offsets, sorted_slot=ss[:TK], slot_pos=sp[:TK],
                   act=act[:TK], o=o[:TK])


def forward_tokens(x, topk_ids, topk_weights, up_proj, down_proj, toks):
    """Rows y[toks] [n,H] float64 from the per-token definition."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(topk_ids)
    g = np.ascontiguousarray(topk_weights, dtype=np.float32)
    up = np.ascontiguousarray(up_proj)
    down = np.ascontiguousarray(down_proj)
    T, H, I, E, K = _shapes(x, ids, up, down)
    toks = np.ascontiguousarray(toks, dtype=np.int64)
    y = np.zeros((max(len(toks), 1), H), np.float64)
    _check(_load().moe_oracle_fwd_tokens(T, H, I, E, K, _dt(x), _p(x), _p(ids), _idt(ids),
                                         _p(g), _p(up), _p(down), _p(toks), len(toks), _p(y)))
    return y[:len(toks)]


def backward(dy, x, topk_ids, topk_weights, up_proj, down_proj):
    """(dx [T,H], d_up [E,H,2I], d_down [E,I,H], d_topk [T,K]) float64."""
    x = np.ascontiguousarray(x)
    dy = np.ascontiguousarray(dy)
    ids = np.ascontiguousarray(topk_ids)
    g = np.ascontiguousarray(topk_weights, dtype=np.float32)
    up = np.ascontiguousarray(up_proj)
    down = np.ascontiguousarray(down_proj)
    T, H, I, E, K = _shapes(x, ids, up, down)
    assert dy.shape == x.shape and dy.dtype == x.dtype
    dx = np.zeros((T, H), np.float64)
    dW1 = np.zeros((E, H, 2 * I), np.float64)
    dW2 = np.zeros((E, I, H), np.float64)
    dg = np.zeros((max(T, 1), K), np.float64)
    _check(_load().moe_oracle_bwd(T, H, I, E, K, _dt(x), _p(dy), _p(x), _p(ids), _idt(ids),
                                  _p(g), _p(up), _p(down), _p(dx), _p(dW1), _p(dW2), _p(dg)))
    return dx, dW1, dW2, dg[:T]


def backward_sampled(dy, x, topk_ids, topk_weights, up_proj, down_proj, toks, w1_cols, w2_rows):
    """Sampled gradients for full-size checks.

    toks: token ids -> dx rows [n,H] and d_topk rows [n,K];
    w1_cols: (e, j) pairs -> d_up[e][:, j] as rows [n1,H];
    w2_rows: (e, i) pairs -> d_down[e][i, :] as rows [n2,H].
    """
    x = np.ascontiguousarray(x)
    dy = np.ascontiguousarray(dy)
    ids = np.ascontiguousarray(topk_ids)
    g = np.ascontiguousarray(topk_weights, dtype=np.float32)
    up = np.ascontiguousarray(up_proj)
    down = np.ascontiguousarray(down_proj)
    T, H, I, E, K = _shapes(x, ids, up, down)
    toks = np.ascontiguousarray(toks, dtype=np.int64)
    w1c = np.ascontiguousarray(np.asarray(w1_cols, dtype=np.int64).reshape(-1, 2))
    w2r = np.ascontiguousarray(np.asarray(w2_rows, dtype=np.int64).reshape(-1, 2))
    n, n1, n2 = len(toks), len(w1c), len(w2r)
    dx = np.zeros((max(n, 1), H), np.float64)
    dg = np.zeros((max(n, 1), K), np.float64)
    d1 = np.zeros((max(n1, 1), H), np.float64)
    d2 = np.zeros((max(n2, 1), H), np.float64)
    _check(_load().moe_oracle_bwd_sampled(T, H, I, E, K, _dt(x), _p(dy), _p(x), _p(ids),
                                          _idt(ids), _p(g), _p(up), _p(down), _p(toks), n,
                                          _p(dx), _p(dg), _p(w1c), n1, _p(d1), _p(w2r), n2,
                                          _p(d2)))
    return dx[:n], dg[:n], d1[:n1], d2[:n2]


# ----------------------------------------------------------------- shared expert
# Issue page, section 6.1 ("shared-expert fused MoE") and the EP overlap issue,
# section 4.3: the shared expert is a SwiGLU feed-forward every token passes
# through, its output added to the combined routed output.  It is the routed
# definition at one expert, K = 1 and gate 1 (the reduction pinned as a dense
# SwiGLU FFN), applied to shared_up [H, 2Is] and shared_down [Is, H].
def _single_expert_route(T):
    return np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32)


def shared_expert(x, shared_up, shared_down):
    """FFN_s(x) [T,H] float64."""
    ids, g = _single_expert_route(np.asarray(x).shape[0])
    return forward(x, ids, g, np.asarray(shared_up)[None], np.asarray(shared_down)[None])


def forward_shared(x, topk_ids, topk_weights, up_proj, down_proj, shared_up, shared_down):
    """y = Σ_k g·FFN_e(x) + FFN_s(x), [T,H] float64."""
    return (forward(x, topk_ids, topk_weights, up_proj, down_proj)
            + shared_expert(x, shared_up, shared_down))


def backward_shared(dy, x, topk_ids, topk_weights, up_proj, down_proj, shared_up, shared_down):
    """(dx, d_up, d_down, d_topk, d_shared_up [H,2Is], d_shared_down [Is,H]) float64."""
    dx, d_up, d_down, d_topk = backward(dy, x, topk_ids, topk_weights, up_proj, down_proj)
    ids, g = _single_expert_route(np.asarray(x).shape[0])
    sdx, s_up, s_down, _ = backward(dy, x, ids, g, np.asarray(shared_up)[None],
                                    np.asarray(shared_down)[None])
    return dx + sdx, d_up, d_down, d_topk, s_up[0], s_down[0]
