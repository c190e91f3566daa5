"""The layer captured in a HIP graph: every replay, with eager work and host
synchronisations between replays, matches the CPU oracle on that replay's
tokens within the layer's tolerance, and equals the eager call on the same
tokens bit for bit (decode-size FP8 and MXFP4, an MXFP8 prefill-tile shape, and
a BF16 shape whose stage 2 cuts its last round into reduction pieces)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def make(dtype, T, H, I, E, k, seed):
    wl = workloads.Workload(f"graph-{dtype}", T, H, I, E, k, dtype, 1.0, 1.0 / np.sqrt(H), 0.05,
                            seed)
    return workloads.generate(wl)


@pytest.mark.parametrize("dtype,T,H,I,E,k,bm", [
    ("fp8", 1, 1024, 1024, 8, 2, 32),      # one token: route and grouping in one launch
    ("fp8", 16, 1024, 1024, 8, 2, 32),     # decode shape: split reductions, one-wave align
    ("bf16", 700, 512, 768, 8, 2, 256),    # stage 2 tail pieces and their reduction
    ("mxfp4", 16, 1024, 1024, 8, 2, 32),   # E2M1 decode: MX token codes, 128-feature stage 1
    ("mxfp8", 300, 512, 512, 8, 2, 128),   # MX prefill tiles with the code tile in LDS
])
def test_graph_replays_match_eager(dtype, T, H, I, E, k, bm):
    inp = make(dtype, T, H, I, E, k, seed=T)
    say(f"graph {dtype} T={T} H={H} I={I} bm={bm}")
    layer = moe.Layer(dtype, dev(inp.w_router), dev(inp.w1), dev(inp.w3), dev(inp.w2),
                      dev(inp.s1), dev(inp.s3), dev(inp.s2), None, k, T, bm)
    x = dev(inp.x)
    graph = layer.capture(x)
    rng = np.random.default_rng(7)
    for rep in range(4):
        # a new batch of tokens: eager reference first, then the replay on the same memory
        xb = (rng.standard_normal((T, H)).astype(np.float32) *
              (1.0 + rep)).astype(np.float32)
        new = dev(workloads.to_bf16_bits(xb))
        ref = host(moe.Layer.__call__(layer, new)).copy()
        torch.cuda.synchronize()
        x.copy_(new)
        graph.replay()
        torch.cuda.synchronize()
        got = host(layer.out)
        batch = workloads.Inputs(inp.wl, workloads.to_bf16_bits(xb), inp.w_router, None, inp.w1,
                                 inp.w3, inp.w2, inp.s1, inp.s3, inp.s2)
        _, o64 = oracle.forward(batch)
        err = rel_err(got, o64)
        say(f"  replay {rep}: max|err|/max|ref| = {err:.3e}")
        assert err <= TOL[dtype], f"replay {rep}: error {err} against the oracle"
        assert np.array_equal(got, ref), f"replay {rep} differs from the eager call"
        # eager work of the program's own between replays
        _ = (new.float() * 2).sum().item()
