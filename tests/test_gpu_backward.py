"""GPU parity of the backward pass (moe_backward) against the oracle's fp64
gradients: dx, dW1, dW3, dW2, dW_r and the router bias, each within
max|err|/max|ref| <= 2e-2 (the bf16 layer's bound: g, u, dg, du and the
weighted output gradient are held in bf16 between the launches, a few bf16
roundings of 2^-9 each), on small and ragged shapes that span several tiles of
every backward kernel, and on the Mixtral expert shape at the BF16 decode batch
(T=16). Repeated calls give the same bits, and so does the backward from the
pre-activations the training forward keeps (moe_stage1_save_preact)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import dev, host, record_error, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
NAMES = ("dx", "dw1", "dw3", "dw2", "dw_router", "dbias")


def run_backward(inp, dout, bm):
    """Gradients with the pre-activations recomputed, twice (the same bits), and with the
    ones the training forward kept (moe_stage1_save_preact: the same bits again)."""
    wl = inp.wl
    w1, w3, w2 = dev(inp.w1), dev(inp.w3), dev(inp.w2)
    layer = moe.Layer("bf16", dev(inp.w_router), w1, w3, w2, None, None, None, dev(inp.bias),
                      wl.k, wl.T, bm, save_preact=True)
    x = dev(inp.x)
    layer(x)
    w2t, w13t = moe.preshuffle_backward(w1, w3, w2)
    del w1, w3, w2
    d = dev(dout)
    args = (x, layer.w_router, layer.ids, layer.w, layer.grp, layer.act, layer.pw, w2t, w13t, d)
    g = moe.backward(*args)
    torch.cuda.synchronize()
    again = moe.backward(*args)
    saved = moe.backward(*args, gu=layer.gu)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g[n], again[n]), f"{n} not reproducible bit for bit"
        assert torch.equal(g[n], saved[n]), f"{n}: saved pre-activations give other bits"
    return {n: host(g[n]) for n in NAMES}


def compare(tag, got, ref, T):
    worst = 0.0
    for n in NAMES:
        r = ref[n]
        scale = np.abs(r).max()
        err = float(np.abs(got[n].astype(np.float64) - r).max() / scale) if scale > 0 else \
            float(np.abs(got[n]).max())
        say(f"  {tag} {n}: max|err|/max|ref| = {err:.3e}")
        record_error(f"{tag} {n}", err, TOL, T, T)
        worst = max(worst, err)
        assert err <= TOL, f"{n}: {err}"
    return worst


def make(T, H, I, E, k, seed, bias=False):
    wl = workloads.Workload(f"bwd-{T}-{H}-{I}-{E}-{k}", T, H, I, E, k, "bf16", 1.0,
                            1.0 / np.sqrt(H), 0.05, seed)
    inp = workloads.generate(wl)
    if bias:
        inp.bias = np.linspace(-0.5, 0.5, E).astype(np.float32)
    rng = np.random.default_rng(seed + 1000)
    dout = workloads.to_bf16_bits(rng.standard_normal((T, H)))
    return inp, dout


@pytest.mark.parametrize("T,H,I,E,k,bm,bias", [
    (33, 256, 384, 8, 2, 32, False),    # decode tiles: reductions split over waves
    (5, 1024, 1024, 8, 2, 32, True),    # few slots: stage-2 reduction split over workgroups
    (200, 512, 512, 8, 2, 128, False),  # 128-row tiles, several per expert
    (700, 256, 256, 8, 2, 256, True),   # block_m 256, several 128-row tiles per expert
    (17, 256, 256, 4, 1, 32, False),    # k = 1
    (9, 256, 256, 1, 1, 32, False),     # E = 1: a plain SwiGLU MLP, no router gradient
    (48, 256, 256, 16, 4, 32, True),    # E = 16, k = 4: finer-grained experts
])
def test_backward_matches_oracle(T, H, I, E, k, bm, bias):
    inp, dout = make(T, H, I, E, k, seed=T + I, bias=bias)
    say(f"backward T={T} H={H} I={I} E={E} k={k} bm={bm}")
    got = run_backward(inp, dout, bm)
    ref = oracle.backward(inp, dout)
    compare(f"bwd-T{T}-H{H}-I{I}-E{E}-k{k}-bm{bm}", got, ref, T)


def test_backward_mixtral_bf16_T16():
    wl = workloads.config(1)
    say(f"{wl.name} backward: generating inputs")
    inp = workloads.generate(wl, threads=16)
    dout = workloads.to_bf16_bits(np.random.default_rng(77).standard_normal((wl.T, wl.H)))
    bm = moe.pick_block_m(wl.T, wl.k, wl.E)
    got = run_backward(inp, dout, bm)
    torch.cuda.empty_cache()
    say(f"{wl.name} backward: oracle")
    ref = oracle.backward(inp, dout)
    compare(f"{wl.name} backward", got, ref, wl.T)
