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
