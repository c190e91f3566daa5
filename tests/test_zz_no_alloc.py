"""moe_stage2_noalloc (the stage-2 entry point that allocates nothing and works in
the library's scratch array) against moe_stage2 with a workspace: identical
output bits on two calls in a row, the second with a smaller batch (and a
different element type), through the C ABI; shapes beyond the scratch array
are rejected on the host with MOE_ERR_WORKSPACE."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import workloads
from mixture_experts_routed_top_amd import _lib
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def stage1_outputs(dtype, T, H, I, E, k, seed):
    wl = workloads.Workload(f"noalloc-{dtype}-{T}", T, H, I, E, k, dtype, 1.0, 1.0 / np.sqrt(H),
                            0.05, seed)
    inp = workloads.generate(wl)
    fp8 = dtype == "fp8"
    x = dev(inp.x)
    ids, w, xq, xs, _ = moe.route(x, dev(inp.w_router), k, fp8=fp8)
    bm = moe.pick_block_m(T, k, E)
    grp = moe.align(ids, E, bm)
    pw = moe.preshuffle(dtype, dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(inp.s1), dev(inp.s3),
                        dev(inp.s2))
    act, amax = moe.stage1(dtype, xq if fp8 else x, xs, pw, grp)
    return act, amax, pw, grp, w


def both(dtype, act, amax, pw, grp, w):
    L = _lib.lib()
    dt = moe._dt(dtype)
    T, k = w.shape
    E, H, I, bm = pw.E, pw.H, pw.I, grp.block_m
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: None if t is None else t.data_ptr()
    ref = moe.stage2(dtype, act, amax, pw, grp, w)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    rc = L.moe_stage2_noalloc(dt, P(act), P(amax), P(pw.w2), P(pw.s2), P(grp.sorted_slot),
                              P(grp.tile_expert), P(grp.total), P(w), T, k, E, H, I, bm, P(out),
                              st)
    assert rc == 0, L.moe_last_error()
    torch.cuda.synchronize()
    return host(ref), host(out)


def test_noalloc_matches_stage2_on_two_calls_the_second_smaller():
    for dtype, T in (("fp8", 200), ("fp8", 17), ("bf16", 5)):
        say(f"no-alloc stage 2: {dtype} T={T}")
        act, amax, pw, grp, w = stage1_outputs(dtype, T, 512, 1024, 8, 2, seed=T)
        ref, got = both(dtype, act, amax, pw, grp, w)
        assert np.array_equal(ref, got), f"{dtype} T={T}: outputs differ"


def test_noalloc_rejects_shapes_beyond_the_scratch_array():
    L = _lib.lib()
    FAKE = 1 << 20  # never dereferenced: the check fails before any launch
    need = L.moe_stage2_workspace_bytes(1, 8192, 2, 8, 4096, 14336, 128)
    assert need > 64 << 20
    rc = L.moe_stage2_noalloc(1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8192, 2, 8, 4096,
                              14336, 128, FAKE, None)
    assert rc == _lib.ERR_WORKSPACE
    assert b"scratch" in L.moe_last_error()
