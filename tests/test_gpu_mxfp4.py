"""GPU parity of the MXFP4 path (E2M1 expert weights, two per byte, with one E8M0
scale code per 32 values along the reduction; tokens and the intermediate MXFP8):
the preshuffled E2M1 fragment layout byte for byte, and stage 1, stage 2 and the
layer against the oracle on small and ragged shapes that exercise every kernel
configuration."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import TOL, bf16_to_f64, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def make(T, H, I, E, k, seed, sigma_w=0.05):
    wl = workloads.Workload("mx4-small", T, H, I, E, k, "mxfp4", 1.0, 1.0 / np.sqrt(H), sigma_w,
                            seed)
    return workloads.generate(wl)


def test_preshuffled_e2m1_layout():
    # fragment (row block, kb) = one 1 KB piece; lane l = row l%32, bytes 16*(l/32) .. +15
    # of the fragment's 32 (64 values); gate and up rows interleaved in 32-row blocks.
    E, H, I = 2, 512, 256
    inp = make(4, H, I, E, 2, seed=3)
    pw = moe.preshuffle("mxfp4", dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(inp.s1),
                        dev(inp.s3), dev(inp.s2))
    torch.cuda.synchronize()
    assert pw.H == H and pw.I == I
    d13 = host(pw.w13).view(np.uint8).reshape(E, 2 * I // 32, H // 64, 64, 16)
    d2 = host(pw.w2).view(np.uint8).reshape(E, H // 32, I // 64, 64, 16)
    for e in range(E):
        for rb in range(2 * I // 32):
            src = inp.w1 if rb % 2 == 0 else inp.w3
            for kb in (0, H // 64 - 1):
                for l in range(64):
                    b0 = kb * 32 + 16 * (l // 32)
                    assert np.array_equal(d13[e, rb, kb, l],
                                          src[e, (rb // 2) * 32 + l % 32, b0:b0 + 16])
        for rb in (0, H // 32 - 1):
            for kb in range(I // 64):
                for l in range(64):
                    b0 = kb * 32 + 16 * (l // 32)
                    assert np.array_equal(d2[e, rb, kb, l], inp.w2[e, rb * 32 + l % 32, b0:b0 + 16])


def run_stages(inp, bm):
    wl = inp.wl
    ids, w, xq, xs, _ = moe.route(dev(inp.x), dev(inp.w_router), wl.k, dev(inp.bias), mx=True)
    grp = moe.align(ids, wl.E, bm)
    pw = moe.preshuffle("mxfp4", dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(inp.s1),
                        dev(inp.s3), dev(inp.s2))
    act, amax = moe.stage1("mxfp4", xq, xs, pw, grp)
    assert amax is None
    out = moe.stage2("mxfp4", act, None, pw, grp, w)
    torch.cuda.synchronize()
    return dict(ids=host(ids), act=host(act), out=host(out))


@pytest.mark.parametrize("T,H,I,E,k,bm", [
    (40, 512, 768, 8, 2, 32),       # 32-row tiles
    (200, 256, 512, 8, 2, 64),      # 64-row tiles
    (300, 512, 512, 8, 2, 128),     # 128-row tiles, 512-feature workgroups in both stages
    (700, 512, 768, 8, 2, 256),     # block_m 256: several 128-row tiles per expert
    (150, 768, 512, 8, 2, 128),     # H % 512 != 0: stage 2 on 2 fragments per wave
    (130, 1024, 768, 6, 3, 64),     # k = 3 over 6 experts, 64-row tiles
    (17, 256, 256, 4, 1, 32),       # k = 1
    (48, 256, 512, 16, 4, 32),      # E = 16, k = 4: finer-grained experts
    (5, 1024, 1024, 8, 2, 32),      # decode: reduction split over waves and workgroups
    (33, 8192, 256, 4, 2, 32),      # largest H: the whole stage-1 code tile
    (6, 256, 16384, 2, 1, 32),      # largest I: the whole stage-2 code tile
    (9, 256, 256, 1, 1, 32),        # E = 1: a plain SwiGLU MLP
])
def test_mx4_stages_match_oracle(T, H, I, E, k, bm):
    inp = make(T, H, I, E, k, seed=T + H)
    say(f"mxfp4 stages T={T} H={H} I={I} E={E} k={k} bm={bm}")
    r = run_stages(inp, bm)
    o = oracle.align(r["ids"], E, bm)
    ss = o["sorted_slot"]
    real = np.nonzero(ss < T * k)[0]
    toks = (ss[real] // k).astype(np.int32)
    exps = r["ids"].ravel()[ss[real]].astype(np.int32)
    ref = oracle.swiglu("mxfp4", inp.x, inp.w1, inp.w3, inp.s1, inp.s3, toks, exps)
    got = bf16_to_f64(r["act"][real])
    e1 = np.abs(got - ref).max() / np.abs(ref).max()
    pad = np.nonzero(ss >= T * k)[0]
    assert np.all(r["act"][pad] == 0)
    _, o64 = oracle.forward(inp)
    e2 = rel_err(r["out"], o64)
    say(f"  stage1 rel err {e1:.3e}  layer rel err {e2:.3e}")
    assert e1 <= 1e-2
    assert e2 <= TOL["mxfp4"]


def test_mx4_stage2_tail_round_in_pieces_and_determinism():
    T, H, I = 2200, 4096, 512
    inp = make(T, H, I, 8, 2, seed=13, sigma_w=0.02)
    say(f"mxfp4 stage-2 tail pieces: T={T} H={H} I={I}")
    r = run_stages(inp, 128)
    r2 = run_stages(inp, 128)
    assert np.array_equal(r["out"], r2["out"])
    rng = np.random.default_rng(2)
    o = oracle.align(r["ids"], 8, 128)
    ss = o["sorted_slot"]
    last = ss[max(0, o["total"] // 128 - 16) * 128:]
    toks = np.unique(np.concatenate([np.unique(last[last < 2 * T] // 2),
                                     rng.choice(T, 32, replace=False)])).astype(np.int32)
    _, o64 = oracle.forward(inp, toks)
    err = rel_err(r["out"][toks], o64)
    say(f"  {toks.size} tokens: rel err {err:.3e}")
    assert err <= TOL["mxfp4"]


def test_mx4_scale_codes_are_applied():
    # W2 block codes + 1 doubles every output exactly (a power-of-two scale change
    # commutes with every rounding on the way)
    inp = make(64, 512, 512, 4, 2, seed=5)
    a = run_stages(inp, 32)["out"]
    inp.s2 = (inp.s2 + 1).astype(np.uint8)
    b = run_stages(inp, 32)["out"]
    assert np.array_equal(bf16_to_f64(b), 2.0 * bf16_to_f64(a))


def test_mx4_sign_nibbles():
    # Flipping the sign bit of every W3 nibble negates u, hence the intermediate and the
    # output, exactly (every rounding on the way is odd). Only the rows the grouping
    # defines are compared: capacity rows past the padded total are never written.
    inp = make(40, 512, 512, 4, 2, seed=8)
    a = run_stages(inp, 32)
    inp.w3 = (inp.w3 ^ 0x88).astype(np.uint8)
    b = run_stages(inp, 32)
    assert np.array_equal(a["ids"], b["ids"])
    n = oracle.align(a["ids"], 4, 32)["total"]
    assert np.array_equal(bf16_to_f64(b["act"][:n]), -bf16_to_f64(a["act"][:n]))
    assert np.array_equal(bf16_to_f64(b["out"]), -bf16_to_f64(a["out"]))
