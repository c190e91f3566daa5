"""GPU parity at the full Mixtral 8x7B expert shape (H=4096, I=14336, E=8, top-2)
in the launch configuration the benchmark times. Routing and grouping are
compared bit for bit on every token; the layer output on a sample of tokens
the oracle computes one by one (covering every expert, the first and the last
token)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import TOL, Uploaded, host, rel_err, sample_tokens, say

pytestmark = pytest.mark.gpu


def check_full(wl, n_sample, inp=None):
    say(f"{wl.name}: generating inputs")
    inp = inp or workloads.generate(wl, threads=16)
    up = Uploaded(inp)
    say(f"{wl.name}: block_m={up.layer.bm}, running")
    out = up.run()
    ids = host(up.layer.ids)
    oid, ow, _ = oracle.route(inp.x, inp.w_router, inp.bias, wl.k)
    assert np.array_equal(ids, oid)
    np.testing.assert_allclose(host(up.layer.w), ow, rtol=1e-6)
    o = oracle.align(oid, wl.E, up.layer.bm)
    n = int(host(up.layer.grp.total)[0])
    assert n == o["total"]
    assert np.array_equal(host(up.layer.grp.sorted_slot)[:n], o["sorted_slot"])
    if wl.dtype == "fp8":
        oq, os_ = oracle.quant_tokens(inp.x)
        assert np.array_equal(host(up.layer.xq), oq) and np.array_equal(host(up.layer.xs), os_)
    if wl.dtype in ("mxfp8", "mxfp4"):
        oq, os_ = oracle.quant_tokens_mx(inp.x)
        assert np.array_equal(host(up.layer.xq), oq) and np.array_equal(host(up.layer.xs), os_)
    toks = sample_tokens(oid, wl.E, n_sample)
    say(f"{wl.name}: oracle on {toks.size} tokens")
    _, o64 = oracle.forward(inp, toks)
    err = rel_err(out[toks], o64)
    say(f"{wl.name}: rel err {err:.3e} (tolerance {TOL[wl.dtype]})")
    assert err <= TOL[wl.dtype]
    again = up.run()
    assert np.array_equal(again, out), "not reproducible bit for bit"
    del up
    torch.cuda.empty_cache()
    return inp


def test_mixtral_bf16_decode_T16():
    check_full(workloads.config(1), 16)


def test_mixtral_fp8_prefill_T8192():
    check_full(workloads.config(2), 48)


def test_mixtral_fp8_decode_sweep():
    base = None
    for T in workloads.DECODE_SWEEP:
        wl = workloads.config(3, T)
        if base is None:
            base = workloads.generate(wl, threads=16)
            inp = base
        else:  # same weights, this batch's tokens
            xi = workloads.generate(wl, weights=False)
            inp = workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2,
                                   base.s1, base.s3, base.s2)
        check_full(wl, min(T, 8), inp)


def test_mixtral_fp8_skewed_T16384():
    check_full(workloads.config(4), 48)


def test_mixtral_mxfp8_prefill_T8192_and_decode_T16():
    base = check_full(workloads.mxfp8(8192), 32)
    wl = workloads.mxfp8(16)
    xi = workloads.generate(wl, weights=False)
    inp = workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2, base.s1,
                           base.s3, base.s2)
    check_full(wl, 8, inp)


def test_mixtral_mxfp4_decode_sweep_and_prefill_T8192():
    # every batch the benchmark times: the decode sweep T = 1 .. 256 (32- and 128-row
    # tiles) and the prefill, on one set of E2M1 weights
    base = None
    for T in workloads.DECODE_SWEEP:
        wl = workloads.mxfp4(T)
        if base is None:
            base = workloads.generate(wl, threads=16)
            inp = base
        else:
            xi = workloads.generate(wl, weights=False)
            inp = workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2,
                                   base.s1, base.s3, base.s2)
        check_full(wl, min(T, 16), inp)
    wl = workloads.mxfp4(8192)
    xi = workloads.generate(wl, weights=False)
    inp = workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2, base.s1,
                           base.s3, base.s2)
    check_full(wl, 32, inp)
