"""The layer captured into a HIP graph (torch.cuda.CUDAGraph over the library's
launches) and replayed: every replay must reproduce the eager result bit for
bit, with eager work and synchronisations between the replays.  The forward
and backward use no memsets, allocations or host synchronisations, so they can
be captured."""

import pytest
import torch

from gpu_util import say, to_device
from synth import Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pipelined", [False, True], ids=["bulk", "pipelined"])
def test_graph_replays_match_eager(gpu_lib, pipelined):
    w = Workload("graph", 500, T=384, H=512, I=256, E=8, K=2)
    d = to_device(make_inputs(w, with_dy=True))
    say(f"[graph] pipelined={pipelined}")

    def step():
        y, saved = gpu_lib.moe_ffn_fwd(d["x"], d["topk_ids"], d["topk_weights"], d["up_proj"],
                                       d["down_proj"], save_for_backward=True,
                                       pipelined=pipelined)
        grads = gpu_lib.moe_ffn_bwd(d["dy"], d["x"], d["topk_ids"], d["topk_weights"],
                                    d["up_proj"], d["down_proj"], saved)
        return (y,) + tuple(grads)

    ref = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for i in range(3):
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), i
        step()  # eager work between replays
        torch.cuda.synchronize()
