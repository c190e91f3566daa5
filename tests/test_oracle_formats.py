"""Pins of the oracle's number formats against torch's casts and brute force."""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3fn_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3fn_decode_all_codes_match_torch():
    ours = oracle.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    ref = torch_e4m3fn_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def _sweep():
    vals = torch_e4m3fn_values()
    fin = np.unique(vals[np.isfinite(vals)])
    mids = (fin[:-1] + fin[1:]) / 2.0  # exact ties between neighbouring codes
    rng = np.random.default_rng(7)
    rand = rng.uniform(-448, 448, 200000)
    small = rng.uniform(-0.05, 0.05, 50000)
    tiny = rng.uniform(-2.0 ** -8, 2.0 ** -8, 50000)
    near = np.concatenate([np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    v = np.concatenate([fin, mids, near, rand, small, tiny, [0.0, -0.0, 448.0, -448.0]])
    v = v.astype(np.float32)
    return v[np.abs(v) <= 448.0]


def test_e4m3fn_encode_matches_torch_cast():
    v = _sweep()
    ours = oracle.f32_to_e4m3fn(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_encode_is_nearest_ties_to_even_bruteforce():
    """Brute force: the code of |x| is the positive finite code nearest to |x|
    (the even code on a tie); the sign bit is x's sign bit."""
    v = _sweep()[::5]
    vals = torch_e4m3fn_values()
    pos = np.arange(0x7F)  # 0x00..0x7E: the non-negative finite codes
    pv = vals[pos]
    ours = oracle.f32_to_e4m3fn(v).astype(np.int64)
    for x, q in zip(v.astype(np.float64), ours):
        d = np.abs(pv - abs(x))
        cand = pos[d == d.min()]
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        assert len(cand) == 1
        expect = int(cand[0]) | (0x80 if np.signbit(x) else 0)
        assert int(q) == expect, (x, q, expect)


def test_e4m3fn_encode_saturates():
    v = np.array([448.0, 460.0, 1e6, -500.0, np.inf, -np.inf], np.float32)
    assert list(oracle.f32_to_e4m3fn(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]


def test_bf16_round_trip_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                  3.3895314e38], np.float32),
    ])
    # exact ties: bf16 value plus half an ulp
    b = torch.from_numpy(v[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties])
    ours = oracle.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy())


def test_bf16_nan_stays_nan():
    v = np.array([np.nan], np.float32)
    assert np.isnan(oracle.bf16_to_f64(oracle.f32_to_bf16(v)))[0]


# --- MX (E8M0 block scale, E4M3 elements) ------------------------------------

def test_e8m0_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def mx_reference(xf32):
    """Block quantisation from numpy's log2 and torch's e4m3fn cast (library routines)."""
    T, H = xf32.shape
    b = xf32.astype(np.float64).reshape(T, H // 32, 32)
    amax = np.abs(b).max(2)
    with np.errstate(divide="ignore"):
        x = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0)
    x = np.clip(x, -127, 127).astype(np.int64)
    r = np.clip(b * np.exp2(-x)[:, :, None], -448, 448).astype(np.float32)
    q = torch.from_numpy(r.reshape(T, H)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, (x + 127).astype(np.uint8)


def _bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _mx_rows():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 256)).astype(np.float32)
    x[1] *= 1e-3
    x[2] *= 300.0
    x[3, :32] = 0.0                                   # an all-zero block
    x[4, 32:64] = np.float32(2.0 ** -130)             # a subnormal block: scale clamps at 2^-127
    x[5, 64:96] = np.linspace(-511.0, 511.0, 32)      # block maximum just under a power of two
    x[6, 96:128] = np.float32(256.0)                  # block maximum exactly a power of two
    x[7] = rng.standard_normal(256).astype(np.float32) * np.float32(2.0 ** 100)
    return _bf16(x)


def test_mx_quant_matches_library_reference():
    xb = _mx_rows()
    q, s = oracle.quant_tokens_mx(xb)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    rq, rs = mx_reference(xf)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)
    assert np.all(s[3, 0] == 127) and np.all(q[3, :32] == 0)
    assert s[4, 1] == 0


def test_mx_quant_closed_forms():
    xb = _mx_rows()
    q, s = oracle.quant_tokens_mx(xb)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vals = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = vals * np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    b = np.abs(xf).reshape(40, 8, 32).max(2)
    big = np.abs(vals).reshape(40, 8, 32).max(2)
    live = (b > 2.0 ** -100)
    # the block maximum lands in [256, 448]: the top binade of e4m3fn (saturating above 448)
    assert np.all((big[live] >= 256) & (big[live] <= 448))
    # relative error of every element at most half an e4m3fn ulp of its binade (2^-4),
    # except the saturated ones (|x| / 2^e in (448, 512))
    scale = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    sat = np.abs(xf) / scale > 448
    norm = (np.abs(xf) / scale >= 2.0 ** -6) & ~sat
    assert np.all(np.abs(deq - xf)[norm] <= 2.0 ** -4 * np.abs(xf)[norm] * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 448 * scale[sat])


def test_mx_quant_is_blockwise_and_scale_equivariant():
    xb = _mx_rows()[8:]
    q, s = oracle.quant_tokens_mx(xb)
    # x * 2^3 (exact in bf16 for these values): same codes, every scale + 3
    x8 = (xb.astype(np.uint32) + (3 << 7)).astype(np.uint16)
    assert np.all((xb & 0x7F80) != 0) and np.all((x8 & 0x7F80) != 0x7F80)
    q8, s8 = oracle.quant_tokens_mx(x8)
    assert np.array_equal(q8, q) and np.array_equal(s8.astype(int), s.astype(int) + 3)
    # changing one block leaves the other blocks' codes and scales alone
    x2 = xb.copy()
    x2[:, 64:96] = _bf16(np.full((xb.shape[0], 32), 1000.0))
    q2, s2 = oracle.quant_tokens_mx(x2)
    keep = np.ones(256, bool)
    keep[64:96] = False
    assert np.array_equal(q2[:, keep], q[:, keep])
    assert np.array_equal(np.delete(s2, 2, axis=1), np.delete(s, 2, axis=1))


# --- E2M1 (MXFP4 elements) ----------------------------------------------------

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX specification's E2M1 values


def test_e2m1_decode_all_codes_match_the_published_table():
    vals = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert list(vals[:8]) == E2M1_TABLE
    assert list(-vals[8:]) == E2M1_TABLE and np.all(np.signbit(vals[8:]))
    # only the low nibble is read
    assert np.array_equal(oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8) | 0xF0), vals)


def test_e2m1_encode_is_nearest_ties_to_even_bruteforce():
    tab = np.array(E2M1_TABLE)
    mids = (tab[:-1] + tab[1:]) / 2
    rng = np.random.default_rng(5)
    v = np.concatenate([tab, mids, np.nextafter(mids, 0), np.nextafter(mids, 9),
                        rng.uniform(0, 6, 20000), [0.0]]).astype(np.float32)
    v = np.concatenate([v, -v])
    ours = oracle.f32_to_e2m1(v).astype(int)
    for x, q in zip(v.astype(np.float64), ours):
        d = np.abs(tab - abs(x))
        cand = np.nonzero(d == d.min())[0]
        if len(cand) > 1:
            cand = cand[cand % 2 == 0]
        assert q == int(cand[0]) | (8 if np.signbit(x) else 0), (x, q)


def test_e2m1_encode_saturates():
    v = np.array([6.0, 6.5, 100.0, -7.0, np.inf], np.float32)
    assert list(oracle.f32_to_e2m1(v)) == [7, 7, 7, 15, 7]


def test_mx4_weight_storage_matches_the_oracle_encoder():
    import workloads
    rng = np.random.default_rng(6)
    a = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    a[3, :32] = 0.0
    packed, s = workloads.quantize_blocks_mx4(a)
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(16, 256)
    scale = oracle.e8m0_to_f64(s).repeat(32, 1)
    ref = oracle.f32_to_e2m1((a / scale).astype(np.float32))  # a / 2^x is exact
    assert np.array_equal(codes, ref)
    assert s[3, 0] == 127
    # block maxima land in the top binade [4, 6] (saturating above 6)
    big = np.abs(oracle.e2m1_to_f64(codes)).reshape(16, 8, 32).max(2)
    live = np.abs(a).reshape(16, 8, 32).max(2) > 0
    assert np.all((big[live] >= 4) & (big[live] <= 6))
