"""GPU parity of the fused launches.

moe_route_align (the router's last workgroup builds the grouping): every output
equals the oracle's routing, token quantisation and grouping bit for bit, on
both fused paths (one wave up to 128 slots, the 256-thread runs up to 2048)
and on the two-launch fallback, and the ticket is left at zero.

moe_stage2 (FP8 requantisation on load, combine by the last workgroup of each
token and feature tile): repeated calls on one workspace give the same bits
(the tickets are left at zero), and the output matches the oracle."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import TOL, Uploaded, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,E,k,bm,quant", [
    (1, 4096, 8, 2, 32, "fp8"),       # decode T=1: one workgroup, one-wave grouping
    (5, 1024, 8, 2, 32, "mx"),
    (64, 512, 8, 2, 32, None),        # 128 slots: the one-wave limit
    (65, 512, 8, 2, 32, "fp8"),       # 130 slots: the runs path on 256 threads
    (256, 4096, 8, 2, 128, "fp8"),    # decode T=256 with 128-row tiles
    (700, 256, 16, 2, 64, "mx"),      # 16 experts (eight counter words)
    (1023, 256, 8, 2, 256, "fp8"),    # 2046 slots: the largest fused grouping
    (300, 256, 8, 8, 32, None),       # 2400 slots: two launches
    (1024, 256, 8, 2, 128, "fp8"),    # T >= 1024: the wave router, then the align kernel
])
def test_route_align_matches_oracle(T, H, E, k, bm, quant):
    rng = np.random.default_rng(T)
    x = workloads.to_bf16_bits(rng.standard_normal((T, H)))
    wr = workloads.to_bf16_bits(rng.standard_normal((E, H)) / np.sqrt(H))
    say(f"route_align T={T} H={H} E={E} k={k} bm={bm} quant={quant}")
    ticket = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rep in range(2):  # the second call reuses the ticket the first left at zero
        ids, w, xq, xs, g = moe.route_align(dev(x), dev(wr), k, E, bm, quant=quant,
                                            ticket=ticket)
        torch.cuda.synchronize()
        assert int(ticket.item()) == 0, "ticket not reset"
        oid, ow, _ = oracle.route(x, wr, None, k)
        assert np.array_equal(host(ids), oid)
        np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=0)
        if quant == "fp8":
            oq, os_ = oracle.quant_tokens(x)
            assert np.array_equal(host(xq), oq) and np.array_equal(host(xs), os_)
        if quant == "mx":
            oq, os_ = oracle.quant_tokens_mx(x)
            assert np.array_equal(host(xq), oq) and np.array_equal(host(xs), os_)
        o = oracle.align(oid, E, bm)
        n = int(host(g.total)[0])
        assert n == o["total"]
        assert np.array_equal(host(g.sorted_slot)[:n], o["sorted_slot"])
        assert np.array_equal(host(g.tile_expert)[:n // bm], o["tile_expert"])
        assert np.array_equal(host(g.count), o["count"])
        assert np.array_equal(host(g.offset), o["offset"])


@pytest.mark.parametrize("dtype,T,H,I,bm", [
    ("fp8", 1, 1024, 1024, 32),      # decode: reduction split over waves and workgroups
    ("fp8", 300, 512, 768, 128),     # 128-row tiles
    ("bf16", 700, 512, 768, 256),    # tail pieces of the last round
    ("mxfp8", 40, 512, 512, 32),
])
def test_stage2_tickets_left_zero(dtype, T, H, I, bm):
    wl = workloads.Workload(f"tickets-{dtype}", T, H, I, 8, 2, dtype, 1.0, 1.0 / np.sqrt(H),
                            0.05, T)
    inp = workloads.generate(wl)
    say(f"stage-2 tickets {dtype} T={T} H={H} I={I} bm={bm}")
    up = Uploaded(inp, bm)
    first = up.run()
    for _ in range(3):
        assert np.array_equal(up.run(), first), "a repeated call differs"
    _, o64 = oracle.forward(inp)
    err = rel_err(first, o64)
    say(f"  max|err|/max|ref| = {err:.3e}")
    assert err <= TOL[dtype]
    # The tickets sit at the end of the workspace: one word per token and feature tile
    # (at least H/512 tiles), then 256 words for the tail tiles, then padding. All of it
    # is zero after every call.
    ws = host(up.layer.ws)
    assert not ws[-(1024 + T * (H // 512) * 4):].any(), "tickets not reset"
