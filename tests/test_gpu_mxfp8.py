"""GPU parity of the MXFP8 path (e4m3fn values, one E8M0 scale code per 32 values
along the reduction): the block quantisation of x bit for bit, the preshuffled
scale codes' layout, and stage 1, stage 2 and the layer against the oracle on
small and ragged shapes that exercise every kernel configuration."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import TOL, bf16_to_f64, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T", [300, 1100])  # one workgroup per token; eight waves per CU
def test_route_mx_codes_bitexact(T):
    rng = np.random.default_rng(21)
    H, E = 4096, 8
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[1] *= 1e-3
    x[2] *= 300.0
    x[3, :32] = 0.0                                  # all-zero block: code 127
    x[4, 32:64] = np.float32(2.0 ** -130)            # subnormal block: code 0
    x[5, 64:96] = np.linspace(-500.0, 500.0, 32)     # saturating block maximum
    x[6, :] = 0.0                                    # an all-zero token
    xb = bf16_bits(x)
    wr = bf16_bits(rng.standard_normal((E, H)) / 64.0)
    for k in (1, 2):
        ids, w, xq, xs, lg = moe.route(dev(xb), dev(wr), k, None, mx=True, want_logits=True)
        ids8, w8, _, _, lg8 = moe.route(dev(xb), dev(wr), k, None, fp8=True, want_logits=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(ids), host(ids8)) and np.array_equal(host(w), host(w8))
        oq, os_ = oracle.quant_tokens_mx(xb)
        assert np.array_equal(host(xs), os_), np.argwhere(host(xs) != os_)[:5]
        assert np.array_equal(host(xq), oq), np.argwhere(host(xq) != oq)[:5]
    assert os_[3, 0] == 127 and os_[4, 1] == 0 and np.all(os_[6] == 127)


def test_preshuffled_mx_layout():
    # Every scale code reaches the slot the header documents: per expert, groups of
    # four 32-row blocks, then fragment kb, then lane l, then the block j; values
    # follow the instruction's K grouping.
    E, H, I = 2, 512, 256
    wl = workloads.Workload("mx-layout", 4, H, I, E, 2, "mxfp8", 1.0, 1.0 / 16, 0.05, 2)
    inp = workloads.generate(wl)
    rng = np.random.default_rng(0)
    s1 = rng.integers(0, 255, inp.s1.shape, dtype=np.uint8)
    s3 = rng.integers(0, 255, inp.s3.shape, dtype=np.uint8)
    s2 = rng.integers(0, 255, inp.s2.shape, dtype=np.uint8)
    pw = moe.preshuffle("mxfp8", dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(s1), dev(s3), dev(s2))
    torch.cuda.synchronize()
    g13, g2 = host(pw.s13), host(pw.s2)

    def expect(rows_of, R, K):
        KB = K // 64
        out = np.empty(E * R * K // 32, np.uint8)
        o = 0
        for e in range(E):
            for g in range(R // 128):
                for kb in range(KB):
                    for l in range(64):
                        for j in range(4):
                            c = (4 * g + j) * 32 + l % 32
                            out[o] = rows_of(e, c)[2 * kb + l // 32]
                            o += 1
        return out

    def w13_row(e, c):
        src = s1 if (c // 32) % 2 == 0 else s3
        return src[e, (c // 64) * 32 + c % 32]

    assert np.array_equal(g13, expect(w13_row, 2 * I, H))
    assert np.array_equal(g2, expect(lambda e, c: s2[e, c], H, I))
    # values: fragment (row block, kb), piece pc, lane l = row l%32, bytes
    # 32*pc + 16*(l/32) .. +15 of the fragment's 64
    d2 = host(pw.w2).view(np.uint8).reshape(E, H // 32, I // 64, 2, 64, 16)
    for e in range(E):
        for rb in (0, H // 32 - 1):
            for kb in (0, I // 64 - 1):
                for pc in range(2):
                    for l in range(64):
                        b0 = kb * 64 + 32 * pc + 16 * (l // 32)
                        assert np.array_equal(d2[e, rb, kb, pc, l], inp.w2[e, rb * 32 + l % 32, b0:b0 + 16])


def make(T, H, I, E, k, seed, sigma_w=0.05):
    wl = workloads.Workload("mx-small", T, H, I, E, k, "mxfp8", 1.0, 1.0 / np.sqrt(H), sigma_w,
                            seed)
    return workloads.generate(wl)


def run_stages(inp, bm):
    wl = inp.wl
    ids, w, xq, xs, _ = moe.route(dev(inp.x), dev(inp.w_router), wl.k, dev(inp.bias), mx=True)
    grp = moe.align(ids, wl.E, bm)
    pw = moe.preshuffle("mxfp8", dev(inp.w1), dev(inp.w3), dev(inp.w2), dev(inp.s1),
                        dev(inp.s3), dev(inp.s2))
    act, amax = moe.stage1("mxfp8", xq, xs, pw, grp)
    assert amax is None
    out = moe.stage2("mxfp8", act, None, pw, grp, w)
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
def test_mx_stages_match_oracle(T, H, I, E, k, bm):
    inp = make(T, H, I, E, k, seed=T + H)
    say(f"mxfp8 stages T={T} H={H} I={I} E={E} k={k} bm={bm}")
    r = run_stages(inp, bm)
    o = oracle.align(r["ids"], E, bm)
    ss = o["sorted_slot"]
    real = np.nonzero(ss < T * k)[0]
    toks = (ss[real] // k).astype(np.int32)
    exps = r["ids"].ravel()[ss[real]].astype(np.int32)
    ref = oracle.swiglu("mxfp8", inp.x, inp.w1, inp.w3, inp.s1, inp.s3, toks, exps)
    got = bf16_to_f64(r["act"][real])
    e1 = np.abs(got - ref).max() / np.abs(ref).max()
    pad = np.nonzero(ss >= T * k)[0]
    assert np.all(r["act"][pad] == 0)
    _, o64 = oracle.forward(inp)
    e2 = rel_err(r["out"], o64)
    say(f"  stage1 rel err {e1:.3e}  layer rel err {e2:.3e}")
    assert e1 <= 1e-2
    assert e2 <= TOL["mxfp8"]


def test_mx_stage2_tail_round_in_pieces_and_determinism():
    T, H, I = 2200, 4096, 512
    inp = make(T, H, I, 8, 2, seed=13, sigma_w=0.02)
    say(f"mxfp8 stage-2 tail pieces: T={T} H={H} I={I}")
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
    assert err <= TOL["mxfp8"]


def test_mx_scale_codes_are_applied():
    # W2 block codes + 1 doubles every output exactly (a power-of-two scale change
    # commutes with every rounding on the way)
    inp = make(64, 512, 512, 4, 2, seed=5)
    a = run_stages(inp, 32)["out"]
    inp.s2 = (inp.s2 + 1).astype(np.uint8)
    b = run_stages(inp, 32)["out"]
    assert np.array_equal(bf16_to_f64(b), 2.0 * bf16_to_f64(a))
