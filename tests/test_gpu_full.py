"""Full-output parity of the HIP path at the study workloads' full sizes.

Every element of y (and, for the forward+backward shapes, of dx, d_up, d_down
and d_topk) is compared with the oracle run on the whole batch, in the launch
configuration the benchmark times: the layer of the HyperMegaMoE issue page
(section 2.1 forward, section 2.2 backward), the five shapes plus the shared
expert variants.  The sampled tests elsewhere check single tokens at these
sizes; these check the whole output.

Tolerance: max|err| / max|ref| <= 1e-2 for bf16 and 1e-5 for fp32, per
tensor.  The issue page's own functional-test bound (rtol = atol = 1e-3 for
bf16, section 7.1) is printed beside it, not gated: an elementwise bf16 output
rounded at 2^-8 relative cannot meet it.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_f64, max_rel_err, say, to_device
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _elementwise_1e3(got, ref) -> float:
    """Fraction of elements outside |got - ref| <= 1e-3 + 1e-3 |ref|."""
    bad = np.abs(got - ref) > 1e-3 + 1e-3 * np.abs(ref)
    return float(bad.mean()) if bad.size else 0.0


def _check(name, what, got, ref, dtype):
    got = host_f64(got) if isinstance(got, torch.Tensor) else got
    err = max_rel_err(got, ref)
    say(f"[full] {name} {what} max_rel_err={err:.3e} "
        f"outside_rtol_atol_1e-3={_elementwise_1e3(got, ref):.3%}")
    assert np.isfinite(got).all(), (name, what)
    assert err <= TOL[dtype], (name, what, err)


def _shared(inp, d):
    if inp.get("shared_up") is None:
        return {}, {}
    return ({"shared_up_proj_weight": d["shared_up"], "shared_down_proj_weight": d["shared_down"]},
            (inp["shared_up"], inp["shared_down"]))


FWD = ["tiny_f32", "prefill_bf16", "skewed_bf16", "decode_bf16", "fwdbwd_bf16",
       "prefill_shared_bf16"]


@pytest.mark.parametrize("name", FWD)
def test_forward_whole_output_full_size(gpu_lib, name):
    w = WORKLOADS[name]
    say(f"[full] generating {name}")
    inp = make_inputs(w, with_dy=False)
    d = to_device(inp)
    sh, sh_host = _shared(inp, d)
    say(f"[full] forward {name} T={w.T} H={w.H} I={w.I} E={w.E} K={w.K} Is={w.Is}")
    y = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                            d["down_proj"], **sh)
    torch.cuda.synchronize()
    y = host_f64(y)
    del d
    torch.cuda.empty_cache()
    say(f"[full] oracle forward {name}")
    args = (inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"], inp["down_proj"])
    ref = oracle.forward_shared(*args, *sh_host) if sh_host else oracle.forward(*args)
    _check(name, "y", y, ref, w.dtype)


@pytest.mark.parametrize("name", ["fwdbwd_bf16", "fwdbwd_shared_bf16"])
def test_backward_whole_output_full_size(gpu_lib, name):
    w = WORKLOADS[name]
    say(f"[full] generating {name}")
    inp = make_inputs(w, with_dy=True)
    d = to_device(inp)
    sh, sh_host = _shared(inp, d)
    say(f"[full] forward+backward {name} T={w.T} H={w.H} I={w.I} E={w.E} K={w.K} Is={w.Is}")
    y, saved = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                   d["down_proj"], save_for_backward=True, **sh)
    grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                d["down_proj"], saved, **sh)
    torch.cuda.synchronize()
    y = host_f64(y)
    grads = [host_f64(g) for g in grads]
    del d, saved
    torch.cuda.empty_cache()
    say(f"[full] oracle forward+backward {name}")
    args = (inp["x"], inp["topk_ids"], inp["topk_weights"], inp["up_proj"], inp["down_proj"])
    if sh_host:
        y_ref = oracle.forward_shared(*args, *sh_host)
        refs = oracle.backward_shared(inp["dy"], *args, *sh_host)
        names = ("dx", "d_up", "d_down", "d_topk", "d_shared_up", "d_shared_down")
    else:
        y_ref = oracle.forward(*args)
        refs = oracle.backward(inp["dy"], *args)
        names = ("dx", "d_up", "d_down", "d_topk")
    _check(name, "y", y, y_ref, w.dtype)
    assert len(grads) == len(refs) == len(names)
    for g, r, n in zip(grads, refs, names):
        _check(name, n, g, r, w.dtype)
