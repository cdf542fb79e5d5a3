"""GPU routing is bit-exact against the oracle's counting sort.

Routing (HyperMegaMoE issue page, section 4.1): counts per expert, prefix-sum
offsets, the permutation of the T*K slots into expert-contiguous order
(stable in slot index) and its inverse.  Integer work, so the comparison is
exact on every array.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from synth import Workload, make_routing

pytestmark = pytest.mark.gpu


def ids_case(name):
    rng = np.random.default_rng(abs(hash(name)) % 2**32)
    if name == "uniform":
        return rng.integers(0, 16, size=(257, 3)).astype(np.int32), 16
    if name == "k1":
        return rng.integers(0, 7, size=(100, 1)).astype(np.int32), 7
    if name == "t1":
        return rng.permutation(64)[:6].astype(np.int32).reshape(1, 6), 64
    if name == "t63":
        return rng.integers(0, 8, size=(63, 2)).astype(np.int32), 8
    if name == "t65":
        return rng.integers(0, 8, size=(65, 2)).astype(np.int32), 8
    if name == "all_one":
        return np.full((300, 4), 5, np.int32), 9
    if name == "empty_ends":
        return rng.integers(1, 15, size=(200, 3)).astype(np.int32), 16  # experts 0 and 15 empty
    if name == "e1":
        return np.zeros((50, 3), np.int32), 1
    if name == "e1024":
        return rng.integers(0, 1024, size=(700, 8)).astype(np.int32), 1024
    if name == "dups_i64":
        return rng.integers(0, 5, size=(40, 4)).astype(np.int64), 5
    if name == "zipf_t8191":
        w = Workload("z", 2, T=8191, H=8, I=8, E=32, K=8, routing="zipf", n_empty=3)
        return make_routing(w)[0], 32
    if name == "big_many_chunks":
        return rng.integers(0, 64, size=(40000, 6)).astype(np.int32), 64
    # launch-shape boundaries: 16 chunks of 512 slots are one block, 17 are two
    if name == "chunks16":
        return rng.integers(0, 40, size=(1024, 8)).astype(np.int32), 40
    if name == "chunks17_i64":
        return rng.integers(0, 40, size=(1025, 8)).astype(np.int64), 40
    if name == "e900_one_block":
        return rng.integers(0, 900, size=(900, 8)).astype(np.int32), 900
    if name == "e1024_many_chunks":
        return rng.integers(0, 1024, size=(3000, 8)).astype(np.int32), 1024
    raise KeyError(name)


CASES = ["uniform", "k1", "t1", "t63", "t65", "all_one", "empty_ends", "e1", "e1024",
         "dups_i64", "zipf_t8191", "big_many_chunks", "chunks16", "chunks17_i64",
         "e900_one_block", "e1024_many_chunks"]


@pytest.mark.parametrize("name", CASES)
def test_route_bit_exact(gpu_lib, name):
    ids, E = ids_case(name)
    say(f"[route] case={name} T={ids.shape[0]} K={ids.shape[1]} E={E} dtype={ids.dtype}")
    counts, offsets, ss, sp, ws = gpu_lib.moe_ffn_route(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    want = oracle.route(ids, E)
    for got, ref, nm in zip((counts, offsets, ss, sp), want,
                            ("counts", "offsets", "sorted_slot", "slot_pos")):
        np.testing.assert_array_equal(got.cpu().numpy(), ref, err_msg=nm)
    assert gpu_lib.read_status(ws) == 0


def test_route_zero_tokens(gpu_lib):
    say("[route] T=0")
    ids = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    counts, offsets, ss, sp, ws = gpu_lib.moe_ffn_route(ids, 8)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8
    assert offsets.cpu().tolist() == [0] * 9


def test_route_flags_out_of_range_ids_without_writing_out_of_bounds(gpu_lib):
    say("[route] bad ids")
    ids = np.random.default_rng(1).integers(0, 6, size=(90, 3)).astype(np.int32)
    ids[10, 1] = 6
    ids[77, 0] = -3
    counts, offsets, ss, sp, ws = gpu_lib.moe_ffn_route(torch.from_numpy(ids).cuda(), 6)
    assert gpu_lib.read_status(ws) == 1
    sp = sp.cpu().numpy()
    assert sp[10 * 3 + 1] == -1 and sp[77 * 3] == -1
    # the valid slots are routed exactly as if the bad ones were absent
    good = np.ones(ids.size, bool)
    good[[31, 231]] = False
    flat = ids.ravel()
    assert counts.cpu().numpy().tolist() == np.bincount(flat[good], minlength=6).tolist()
    n_valid = int(offsets.cpu()[-1])
    assert n_valid == ids.size - 2
    want_sorted = np.nonzero(good)[0][np.argsort(flat[good], kind="stable")]
    np.testing.assert_array_equal(ss.cpu().numpy()[:n_valid], want_sorted)


@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_route_flags_bad_ids_in_multi_block_launch(gpu_lib, dtype):
    # more than 16 chunks: the bad-id flags of every chunk reach the status word
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 24, size=(3000, 4)).astype(dtype)
    ids[2999, 3] = 24
    ids[1500, 0] = -1
    say(f"[route] bad ids, multi-block, {np.dtype(dtype).name}")
    counts, offsets, ss, sp, ws = gpu_lib.moe_ffn_route(torch.from_numpy(ids).cuda(), 24)
    assert gpu_lib.read_status(ws) == 1
    flat = ids.ravel()
    good = (flat >= 0) & (flat < 24)
    sp = sp.cpu().numpy()
    assert (sp[~good] == -1).all()
    n_valid = int(offsets.cpu()[-1])
    assert n_valid == int(good.sum())
    want_sorted = np.nonzero(good)[0][np.argsort(flat[good], kind="stable")]
    np.testing.assert_array_equal(ss.cpu().numpy()[:n_valid], want_sorted)
    np.testing.assert_array_equal(sp[want_sorted], np.arange(n_valid))


def test_route_is_deterministic(gpu_lib):
    ids, E = ids_case("big_many_chunks")
    say("[route] determinism")
    t = torch.from_numpy(ids).cuda()
    a = gpu_lib.moe_ffn_route(t, E)
    b = gpu_lib.moe_ffn_route(t, E)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)
