"""GPU parity at the full Mixtral 8x7B expert shape (H=4096, I=14336, E=8, top-2)
in the launch configuration the benchmark times. Routing and grouping are
compared bit for bit on every token. The layer output is compared element by
element with the oracle on every token of the decode batches (T <= 256), and at
prefill sizes on tokens chosen so that every live row tile of both GEMM stages
holds at least one compared slot (cover_tokens): each compared slot's output
row spans all of stage 2's feature tiles, including the row tiles of the last
round that stage 2 cuts into reduction pieces. Each case's max|err|/max|ref|
goes to the parity log (gpu_util.ERROR_LOG)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (TOL, Uploaded, cover_tokens, host, live_row_tiles, record_error, rel_err,
                      say)

pytestmark = pytest.mark.gpu


def check_full(wl, inp=None, all_tokens=None):
    say(f"{wl.name}: generating inputs")
    inp = inp or workloads.generate(wl, threads=16)
    up = Uploaded(inp)
    bm = up.layer.bm
    say(f"{wl.name}: block_m={bm}, running")
    out = up.run()
    ids = host(up.layer.ids)
    oid, ow, _ = oracle.route(inp.x, inp.w_router, inp.bias, wl.k)
    assert np.array_equal(ids, oid)
    np.testing.assert_allclose(host(up.layer.w), ow, rtol=1e-6)
    o = oracle.align(oid, wl.E, bm)
    n = int(host(up.layer.grp.total)[0])
    assert n == o["total"]
    assert np.array_equal(host(up.layer.grp.sorted_slot)[:n], o["sorted_slot"])
    assert np.array_equal(host(up.layer.grp.tile_expert)[:n // bm], o["tile_expert"])
    assert np.array_equal(host(up.layer.grp.count), o["count"])
    if wl.dtype == "fp8":
        oq, os_ = oracle.quant_tokens(inp.x)
        assert np.array_equal(host(up.layer.xq), oq) and np.array_equal(host(up.layer.xs), os_)
    if wl.dtype in ("mxfp8", "mxfp4"):
        oq, os_ = oracle.quant_tokens_mx(inp.x)
        assert np.array_equal(host(up.layer.xq), oq) and np.array_equal(host(up.layer.xs), os_)
    if all_tokens is None:
        all_tokens = wl.T <= 256
    toks = (np.arange(wl.T, dtype=np.int32) if all_tokens else cover_tokens(oid, wl.E, bm))
    tiles = live_row_tiles(oid, wl.E, bm)
    say(f"{wl.name}: oracle on {toks.size} of {wl.T} tokens ({tiles} live row tiles)")
    _, o64 = oracle.forward(inp, toks)
    err = rel_err(out[toks], o64)
    say(f"{wl.name}: rel err {err:.3e} (tolerance {TOL[wl.dtype]})")
    record_error(wl.name, err, TOL[wl.dtype], int(toks.size), wl.T, block_m=bm,
                 live_row_tiles=tiles)
    assert err <= TOL[wl.dtype]
    again = up.run()
    assert np.array_equal(again, out), "not reproducible bit for bit"
    del up
    torch.cuda.empty_cache()
    return inp


def with_tokens(wl, base):
    """Inputs of workload wl that share base's weights (this batch's own tokens)."""
    xi = workloads.generate(wl, weights=False)
    return workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2, base.s1,
                            base.s3, base.s2)


def test_mixtral_bf16_decode_T16():
    check_full(workloads.config(1))


def test_mixtral_fp8_prefill_T8192():
    check_full(workloads.config(2))


def test_mixtral_fp8_decode_sweep():
    base = None
    for T in workloads.DECODE_SWEEP:
        wl = workloads.config(3, T)
        if base is None:
            base = inp = workloads.generate(wl, threads=16)
        else:
            inp = with_tokens(wl, base)
        check_full(wl, inp)


def test_mixtral_fp8_skewed_T16384():
    check_full(workloads.config(4))


def test_mixtral_mxfp8_prefill_T8192_and_decode_T16():
    base = check_full(workloads.mxfp8(8192))
    check_full(workloads.mxfp8(16), with_tokens(workloads.mxfp8(16), base))


def test_mixtral_mxfp4_decode_sweep_and_prefill_T8192():
    # every batch the benchmark times: the decode sweep T = 1 .. 256 (32- and 128-row
    # tiles) and the prefill, on one set of E2M1 weights
    base = None
    for T in workloads.DECODE_SWEEP:
        wl = workloads.mxfp4(T)
        if base is None:
            base = inp = workloads.generate(wl, threads=16)
        else:
            inp = with_tokens(wl, base)
        check_full(wl, inp)
    check_full(workloads.mxfp4(8192), with_tokens(workloads.mxfp4(8192), base))
