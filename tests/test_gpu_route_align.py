"""GPU parity of moe_route_align (routing and grouping in one call, one launch for a
single token with H <= 4096): every output bit for bit equal to
moe_route / moe_route_mx followed by moe_align, and the ids, logits, token codes and
grouping equal to the oracle's."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

CASES = [
    # T, H, E, k, quantisation, bias, block_m
    # one launch (T = 1, H <= 4096)
    (1, 4096, 8, 2, "fp8", False, 32),     # the Mixtral decode shape
    (1, 4096, 8, 2, "mx", True, 32),
    (1, 4096, 8, 2, "none", False, 128),   # bf16 layer: no token quantisation
    (1, 2048, 64, 8, "fp8", True, 64),     # 8 slots over 64 experts
    (1, 4096, 16, 4, "fp8", True, 32),     # two experts per wave
    (1, 512, 6, 3, "mx", False, 32),
    (1, 256, 1, 1, "fp8", False, 256),
    # the two calls' launches
    (1, 8192, 8, 2, "fp8", False, 32),     # H > 4096
    (2, 4096, 8, 2, "fp8", True, 32),
    (4, 4096, 8, 2, "mx", False, 32),
    (4, 2048, 64, 8, "fp8", True, 64),
    (33, 1024, 8, 2, "mx", False, 32),
]


def inputs(T, H, E, seed):
    rng = np.random.default_rng(seed)
    x = workloads.to_bf16_bits(rng.standard_normal((T, H)))
    wr = workloads.to_bf16_bits(rng.standard_normal((E, H)) / 16)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    return x, wr, bias


def bits(t):
    return host(t).view(np.uint8) if t is not None else None


@pytest.mark.parametrize("T,H,E,k,quant,use_bias,bm", CASES)
def test_route_align_matches_separate_calls_and_oracle(T, H, E, k, quant, use_bias, bm):
    say(f"route_align T={T} H={H} E={E} k={k} {quant} bias={use_bias} bm={bm}")
    x, wr, bias = inputs(T, H, E, seed=T * 1000 + H + E)
    b = bias if use_bias else None
    fp8, mx = quant == "fp8", quant == "mx"
    ids, w, xq, xs, lg, g = moe.route_align(dev(x), dev(wr), k, bm, dev(b), fp8=fp8, mx=mx,
                                            want_logits=True)
    ids2, w2, xq2, xs2, lg2 = moe.route(dev(x), dev(wr), k, dev(b), fp8=fp8, mx=mx,
                                        want_logits=True)
    g2 = moe.align(ids2, E, bm)
    torch.cuda.synchronize()
    # the separate calls, bit for bit
    for a, c in ((ids, ids2), (w, w2), (lg, lg2), (xq, xq2), (xs, xs2)):
        assert (a is None) == (c is None)
        if a is not None:
            assert np.array_equal(bits(a), bits(c))
    n = int(host(g.total)[0])
    assert n == int(host(g2.total)[0])
    assert np.array_equal(host(g.sorted_slot)[:n], host(g2.sorted_slot)[:n])
    assert np.array_equal(host(g.tile_expert)[: n // bm], host(g2.tile_expert)[: n // bm])
    assert np.array_equal(host(g.count), host(g2.count))
    assert np.array_equal(host(g.offset), host(g2.offset))
    # the oracle
    oid, ow, olg = oracle.route(x, wr, b, k)
    assert np.array_equal(host(lg), olg)
    assert np.array_equal(host(ids), oid)
    np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=1e-12)
    if fp8:
        oq, os_ = oracle.quant_tokens(x)
        assert np.array_equal(host(xq), oq) and np.array_equal(host(xs), os_)
    if mx:
        oq, os_ = oracle.quant_tokens_mx(x)
        assert np.array_equal(host(xq), oq) and np.array_equal(host(xs), os_)
    o = oracle.align(oid, E, bm)
    assert n == o["total"]
    assert np.array_equal(host(g.sorted_slot)[:n], o["sorted_slot"])
    assert np.array_equal(host(g.tile_expert)[: n // bm], o["tile_expert"])
    assert np.array_equal(host(g.count), o["count"])
    assert np.array_equal(host(g.offset), o["offset"])


def test_route_align_repeated_calls_reuse_buffers():
    """A decode loop: the same output buffers, new tokens each call (the grouping of
    the previous call must not leak into the next)."""
    H, E, k, bm = 4096, 8, 2, 32
    rng = np.random.default_rng(7)
    wr = workloads.to_bf16_bits(rng.standard_normal((E, H)) / 16)
    inp = workloads.generate(workloads.config(3, 1), weights=False)
    layer_x = [inp.x] + [workloads.to_bf16_bits(rng.standard_normal((1, H))) for _ in range(3)]
    for i, x in enumerate(layer_x):
        say(f"route_align decode step {i}")
        ids, w, xq, xs, lg, g = moe.route_align(dev(x), dev(wr), k, bm, fp8=True)
        torch.cuda.synchronize()
        oid, _, _ = oracle.route(x, wr, None, k)
        o = oracle.align(oid, E, bm)
        n = int(host(g.total)[0])
        assert np.array_equal(host(ids), oid)
        assert n == o["total"] and np.array_equal(host(g.sorted_slot)[:n], o["sorted_slot"])
