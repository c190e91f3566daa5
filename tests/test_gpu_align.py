"""GPU parity of moe_align: every output bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import workloads
import oracle
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def ids_for(T, k, E, seed, skew=None):
    rng = np.random.default_rng(seed)
    if skew is None:
        return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    p = np.asarray(skew, float)
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False, p=p / p.sum())
    return out


def check(ids, E, bm):
    T, k = ids.shape
    say(f"align parity T={T} k={k} E={E} bm={bm}")
    g = moe.align(dev(ids), E, bm)
    torch.cuda.synchronize()
    o = oracle.align(ids, E, bm)
    n = int(host(g.total)[0])
    assert n == o["total"]
    assert np.array_equal(host(g.sorted_slot)[:n], o["sorted_slot"])
    assert np.array_equal(host(g.tile_expert)[: n // bm], o["tile_expert"])
    assert np.array_equal(host(g.count), o["count"])
    assert np.array_equal(host(g.offset), o["offset"])


@pytest.mark.parametrize("T,k,E,bm", [(32, 2, 8, 32), (1, 2, 8, 32), (16, 2, 8, 32),
                                      (8192, 2, 8, 128), (8192, 2, 8, 256), (16384, 2, 8, 256),
                                      (257, 3, 64, 64), (1000, 1, 4, 32), (2049, 8, 8, 32),
                                      (64, 2, 8, 128),
                                      # around the one-wave path's limit of 128 slots
                                      (64, 2, 8, 32), (129, 1, 8, 64), (32, 2, 64, 32),
                                      (33, 1, 1, 256), (65, 1, 8, 32), (128, 1, 8, 32),
                                      (256, 1, 8, 32), (100, 2, 12, 32),
                                      # the per-thread-run path (128 < S <= 32768, E <= 16)
                                      # and the chunked path beyond it
                                      (1024, 2, 8, 32), (2049, 1, 8, 64),
                                      (1025, 2, 16, 64), (3000, 2, 64, 64),
                                      (20000, 2, 8, 128)])
def test_align_uniform(T, k, E, bm):
    check(ids_for(T, k, E, T + bm), E, bm)


def test_align_skewed_and_degenerate():
    check(ids_for(5000, 2, 8, 1, skew=[40, 10, 10, 10, 10, 10, 1, 1]), 8, 256)
    one = np.zeros((300, 1), np.int32)  # every slot on expert 0
    check(one, 8, 32)
    last = np.full((33, 1), 7, np.int32)
    check(last, 8, 32)


def test_align_rejects_out_of_range_ids_on_device():
    ids = np.zeros((10, 2), np.int32)
    ids[3, 1] = 8
    g = moe.align(dev(ids), 8, 32)
    torch.cuda.synchronize()
    assert int(host(g.total)[0]) == 0


@pytest.mark.parametrize("dtype", ["fp8", "mxfp8", "mxfp4"])
def test_empty_grouping_gives_zero_output(dtype):
    # stages run on the empty grouping of invalid ids: stage 2's output is all zero
    T, H, I, E, k = 10, 256, 256, 8, 2
    wl = workloads.Workload("empty", T, H, I, E, k, dtype, 1.0, 1.0 / 16.0, 0.05, 9)
    inp = workloads.generate(wl)
    ids = np.zeros((T, k), np.int32)
    ids[0, 0] = E  # out of range
    g = moe.align(dev(ids), E, 32)
    pw = moe.preshuffle(dtype, dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(inp.s1), dev(inp.s3),
                        dev(inp.s2))
    mx = dtype != "fp8"
    _, _, xq, xs, _ = moe.route(dev(inp.x), dev(inp.w_router), k, fp8=not mx, mx=mx)
    act, amax = moe.stage1(dtype, xq, xs, pw, g)
    w = torch.full((T, k), 0.5, dtype=torch.float32, device="cuda")
    out = moe.stage2(dtype, act, amax, pw, g, w)
    torch.cuda.synchronize()
    assert np.all(host(out) == 0)
