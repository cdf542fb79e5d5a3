"""Seeded synthetic inputs for the MoE expert-FFN layer.

This module only draws random numbers and shapes them; it holds none of the
layer's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path consume
the exact bits produced here.

Recipe (one ``numpy.random.SeedSequence([cfg_id, tensor_id, part])`` per tensor
slice, PCG64 bit generator):

* ``x``            ~ N(0, 1), shape [T, H]
* ``up_proj``      ~ N(0, 1/sqrt(H)), shape [E, H, 2I]   (fan_in = H)
* ``down_proj``    ~ N(0, 1/sqrt(I)), shape [E, I, H]    (fan_in = I)
* ``dy``           ~ N(0, 1), shape [T, H]
* ``shared_up``    ~ N(0, 1/sqrt(H)), shape [H, 2·Is]  (workloads with a shared expert)
* ``shared_down``  ~ N(0, 1/sqrt(Is)), shape [Is, H]
* routing "uniform": router logits ~ N(0, 1) [T, E]; ``topk_ids`` are the K
  largest logits of each token in descending order (ties: lower expert id
  first), ``topk_weights`` the softmax over those K logits.
* routing "replace": ids uniform on [0, E) with replacement (duplicate experts
  inside a token), gates the softmax of K N(0,1) draws.
* routing "zipf": Gumbel-top-K (Plackett-Luce) sampling, the logit of the
  expert holding popularity rank r is ``log p_r + Gumbel(0,1)`` with
  ``p_r ∝ r^-s``; the last ``n_empty`` ranks get -inf so those experts stay
  empty; ranks map to expert ids through a seeded permutation.

Floating point tensors are drawn in fp32 and rounded to bf16 with
round-to-nearest-even where the workload is bf16.  bf16 arrays are carried as
``numpy.uint16`` bit patterns.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "make_inputs",
    "make_routing",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "host_threads",
]

# tensor ids inside one workload's seed space
_TID_X, _TID_W1, _TID_W2, _TID_LOGITS, _TID_DY, _TID_PERM, _TID_GUMBEL, _TID_SW1, _TID_SW2 = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic MoE-FFN problem."""

    name: str
    cfg_id: int
    T: int
    H: int
    I: int
    E: int
    K: int
    dtype: str = "bf16"  # "bf16" or "f32": x, weights, y and gradients
    routing: str = "uniform"  # "uniform" or "zipf"
    zipf_s: float = 1.2
    n_empty: int = 0
    backward: bool = False
    Is: int = 0  # intermediate width of the shared expert (0: none)

    @property
    def TK(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def fwd_flops(self) -> float:
        """Algorithmic forward flops: 2*TK*H*2I (up) + 2*TK*I*H (down), plus
        6*T*H*Is for a shared expert."""
        return 6.0 * self.T * self.H * (self.K * self.I + self.Is)

    def bwd_flops(self) -> float:
        return 12.0 * self.T * self.H * (self.K * self.I + self.Is)


# The five workloads of the study: a tiny fp32 case, a prefill shape, a
# skewed prefill shape with Zipf popularity and forced-empty experts, a
# weight-streaming decode shape and a forward+backward shape.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 0, T=256, H=256, I=512, E=8, K=2, dtype="f32"),
        Workload("prefill_bf16", 1, T=4096, H=2048, I=1408, E=64, K=6),
        Workload("skewed_bf16", 2, T=8192, H=7168, I=2048, E=32, K=8, routing="zipf",
                 zipf_s=1.2, n_empty=3),
        Workload("decode_bf16", 3, T=128, H=7168, I=2048, E=32, K=8),
        Workload("fwdbwd_bf16", 4, T=4096, H=4096, I=1536, E=16, K=4, backward=True),
        # the prefill and forward+backward shapes with a shared expert of width
        # 2I and I (the pages give no size; these are common choices)
        Workload("prefill_shared_bf16", 5, T=4096, H=2048, I=1408, E=64, K=6, Is=2816),
        Workload("fwdbwd_shared_bf16", 6, T=4096, H=4096, I=1536, E=16, K=4, backward=True,
                 Is=1536),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF))
    return (r >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _normal_slices(shape, std: float, dtype: str, key, threads: int | None = None):
    """Draw N(0, std) of `shape`; slice i along dim 0 uses its own stream key+(i,)."""
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty(shape, dtype=out_dtype)
    n0 = shape[0]

    def fill(i):
        tmp = _rng(*key, i).standard_normal(shape[1:], dtype=np.float32)
        if std != 1.0:
            tmp *= np.float32(std)
        out[i] = bf16_bits_from_f32(tmp) if dtype == "bf16" else tmp

    threads = threads or min(16, host_threads())
    if n0 * int(np.prod(shape[1:])) < (1 << 22) or threads == 1:
        for i in range(n0):
            fill(i)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n0)))
    return out


def _topk_desc(logits: np.ndarray, K: int) -> np.ndarray:
    # stable sort of the negated logits: descending, ties -> lower expert id
    return np.argsort(-logits, axis=1, kind="stable")[:, :K].astype(np.int32)


def _softmax_rows(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float64)
    m = v.max(axis=1, keepdims=True)
    e = np.exp(v - m)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def make_routing(w: Workload, seed: int = 0):
    """Return (topk_ids int32 [T,K], topk_weights fp32 [T,K], logits fp32 [T,E])."""
    T, E, K = w.T, w.E, w.K
    if w.routing == "replace":
        # ids drawn with replacement (duplicates inside a token allowed)
        rng = _rng(w.cfg_id, _TID_LOGITS, seed)
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
        sel = rng.standard_normal((T, K), dtype=np.float32)
        return ids, _softmax_rows(sel) if T else sel, None
    if K > E:
        raise ValueError("K must not exceed E for distinct top-k routing")
    if w.routing == "uniform":
        logits = _rng(w.cfg_id, _TID_LOGITS, seed).standard_normal((T, E), dtype=np.float32)
    elif w.routing == "zipf":
        n_live = E - w.n_empty
        if K > n_live:
            raise ValueError("K exceeds the number of non-empty experts")
        ranks = np.arange(1, E + 1, dtype=np.float64)
        logp = -w.zipf_s * np.log(ranks)
        logp -= np.log(np.exp(logp[:n_live]).sum())
        logp[n_live:] = -np.inf
        perm = _rng(w.cfg_id, _TID_PERM, seed).permutation(E)  # rank r -> expert perm[r]
        logp_by_expert = np.empty(E)
        logp_by_expert[perm] = logp
        g = _rng(w.cfg_id, _TID_GUMBEL, seed).gumbel(size=(T, E))
        logits = (logp_by_expert[None, :] + g).astype(np.float32)
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    ids = _topk_desc(logits, K)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    gates = _softmax_rows(sel)
    return ids, gates, logits


def make_inputs(w: Workload, seed: int = 0, with_dy: bool | None = None, threads=None):
    """All inputs of one workload as host numpy arrays (bf16 as uint16 bits).

    Returns a dict with x [T,H], topk_ids [T,K] int32, topk_weights [T,K] fp32,
    up_proj [E,H,2I], down_proj [E,I,H] and, for backward workloads, dy [T,H].
    """
    T, H, I, E = w.T, w.H, w.I, w.E
    out = {}
    out["x"] = _normal_slices((max(T, 1), H), 1.0, w.dtype, (w.cfg_id, _TID_X, seed),
                              threads)[:T]
    out["up_proj"] = _normal_slices((E, H, 2 * I), 1.0 / np.sqrt(H), w.dtype,
                                    (w.cfg_id, _TID_W1, seed), threads)
    out["down_proj"] = _normal_slices((E, I, H), 1.0 / np.sqrt(I), w.dtype,
                                      (w.cfg_id, _TID_W2, seed), threads)
    ids, gates, _ = make_routing(w, seed)
    out["topk_ids"] = ids
    out["topk_weights"] = gates
    if w.Is:
        out["shared_up"] = _normal_slices((H, 2 * w.Is), 1.0 / np.sqrt(H), w.dtype,
                                          (w.cfg_id, _TID_SW1, seed), threads)
        out["shared_down"] = _normal_slices((w.Is, H), 1.0 / np.sqrt(w.Is), w.dtype,
                                            (w.cfg_id, _TID_SW2, seed), threads)
    if with_dy is None:
        with_dy = w.backward
    if with_dy:
        out["dy"] = _normal_slices((max(T, 1), H), 1.0, w.dtype, (w.cfg_id, _TID_DY, seed),
                                   threads)[:T]
    return out
