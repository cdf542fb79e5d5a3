"""Helpers shared by the GPU tests: host<->device conversion and error measures."""

import sys

import numpy as np
import torch


def dev_tensor(a: np.ndarray, device="cuda"):
    """numpy (bf16 as uint16 bits, or fp32/int) -> device tensor with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_device(inp: dict, device="cuda"):
    return {k: dev_tensor(v, device) for k, v in inp.items() if v is not None}


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (the parity measure for floating-point outputs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def say(*args):
    """Name the case before a GPU step, flushed, so a crash still tells which one."""
    print(*args, flush=True)
    sys.stdout.flush()


TOL = {"bf16": 1e-2, "f32": 1e-5}
