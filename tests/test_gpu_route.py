"""GPU parity of moe_route: ids, logits, FP8 codes and scales bit-exact against
the oracle; routing weights within 1e-6 relative (or 1e-12 absolute for weights
that are themselves tiny)."""
import json
import os

import numpy as np
import pytest
import torch

import mixture_experts_routed_top_amd as moe
import oracle
import workloads
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_route(x, wr, bias, k, fp8=True, tag=""):
    say(f"route parity {tag}: T={x.shape[0]} H={x.shape[1]} E={wr.shape[0]} k={k}")
    ids, w, xq, xs, lg = moe.route(dev(x), dev(wr), k, dev(bias), fp8=fp8, want_logits=True)
    torch.cuda.synchronize()
    oid, ow, olg = oracle.route(x, wr, bias, k)
    g_lg = host(lg)
    assert np.array_equal(g_lg, olg), f"logits differ at {np.argwhere(g_lg != olg)[:5]}"
    assert np.array_equal(host(ids), oid)
    # expf's error grows with |argument| (about |l_j - l_0| ulps), so a weight far below
    # the largest (logit gaps of tens, from rows spanning many binades) is held to an
    # absolute 1e-12, far below what a bf16 output can show
    np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=1e-12)
    if fp8:
        oq, os_ = oracle.quant_tokens(x)
        assert np.array_equal(host(xs), os_)
        gq = host(xq)
        bad = np.argwhere(gq != oq)
        assert bad.size == 0, f"{len(bad)} x_q codes differ, first {bad[:5]}"
    return host(ids)


def test_route_tiny_bf16():
    inp = workloads.generate(workloads.config(0), weights=False)
    check_route(inp.x, inp.w_router, None, 2, fp8=False, tag="tiny")
    for k in (1, 3, 8):
        check_route(inp.x, inp.w_router, None, k, tag=f"tiny k={k}")


def test_route_mixtral_prefill_fp8():
    inp = workloads.generate(workloads.config(2), weights=False)
    check_route(inp.x, inp.w_router, None, 2, tag="mixtral fp8 T=8192")


def test_route_skewed_bias():
    wl = workloads.config(4)
    inp = workloads.generate(wl, weights=False)
    ids = check_route(inp.x, inp.w_router, inp.bias, 2, tag="skewed T=16384")
    share = np.bincount(ids.ravel(), minlength=8) / ids.size
    assert 0.39 <= share[0] <= 0.41 and share[6] < 0.03 and share[7] < 0.03


def test_route_canonical_order_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "canonical_logit.json")))
    H = g["H"]
    x = np.zeros((1, H), np.float32)
    w = np.zeros((2, H), np.float32)
    for h, xv, wv in g["nonzero"]:
        x[0, h], w[0, h] = xv, wv
    xb, wb = workloads.to_bf16_bits(x), workloads.to_bf16_bits(w)
    _, _, _, _, lg = moe.route(dev(xb), dev(wb), 1, want_logits=True)
    assert float(host(lg)[0, 0]) == g["expected_logit"]


def test_route_ties_zero_rows_and_wide_E():
    rng = np.random.default_rng(4)
    H, E = 256, 64
    wr = workloads.to_bf16_bits(rng.standard_normal((E, H)) / 16)
    wr[9] = wr[2]
    wr[40] = wr[2]
    x = workloads.to_bf16_bits(rng.standard_normal((70, H)))
    x[5] = 0
    x[6] = 0x8000  # -0.0
    ids = check_route(x, wr, None, 8, tag="E=64 k=8 ties")
    assert list(ids[5]) == list(range(8))
    check_route(x, wr, None, 1, tag="E=64 k=1")
    check_route(x[:, :128].copy(), wr[:1, :128].copy(), None, 1, tag="E=1")


@pytest.mark.parametrize("T,H,E,k,bias", [
    (1037, 4096, 8, 2, True),   # ragged: the last wave's second row is past T
    (2051, 2048, 6, 3, False),  # E < 8, two workgroups per CU
    (4133, 3072, 8, 1, True),   # H not a multiple of 512: lanes past the row in the last chunk
    (9000, 4096, 8, 2, False),  # several passes per wave (row prefetch)
])
def test_route_large_batches_with_zeros_and_binades(T, H, E, k, bias):
    """The large-batch launch shape (T >= 1024, E <= 8): rows of normal values, rows
    spanning many binades, zero rows of both signs and rows with scattered zeros; ids,
    logits, codes and scales bit-exact."""
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H)).astype(np.float32)
    m = rng.uniform(1.0, 2.0, (64, H)) * np.exp2(rng.integers(-140, 11, (64, H)).astype(np.float64))
    x[100:164] = (rng.choice([-1.0, 1.0], (64, H)) * m).astype(np.float32)
    x[7] = 0.0
    x[T - 1, ::3] = 0.0
    xb = workloads.to_bf16_bits(x)
    xb[8] = 0x8000  # -0.0
    xb[9, ::5] = 0x8000
    wr = workloads.to_bf16_bits(rng.standard_normal((E, H)) / 64)
    b = np.linspace(-0.3, 0.3, E).astype(np.float32) if bias else None
    check_route(xb, wr, b, k, tag=f"large batch T={T} H={H} E={E}")


def test_fp8_conversion_of_every_bf16_value_in_range():
    """Rows holding every bf16 value in [-448, 448] (plus 448 to fix the scale at 1):
    the device e4m3fn conversion must equal the oracle's nearest-even rounding."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    vals = b[keep]
    H = 4096
    per = H - 1
    rows = -(-vals.size // per)
    x = np.zeros((rows, H), np.uint16)
    flat = np.zeros(rows * per, np.uint16)
    flat[: vals.size] = vals
    x[:, :per] = flat.reshape(rows, per)
    x[:, per] = 0x43E0  # 448.0
    wr = workloads.to_bf16_bits(np.ones((2, H)) / H)
    check_route(x, wr, None, 1, tag="all bf16 codes")


def test_fp8_quantisation_over_many_binades():
    """Rows whose values span 2^-140 .. 2^10 (bf16 normals and subnormals, both signs,
    zeros of both signs): codes and scales bit-exact against the oracle's fp32 divide."""
    rng = np.random.default_rng(11)
    T, H = 64, 4096
    mant = rng.uniform(1.0, 2.0, (T, H))
    expo = rng.integers(-140, 11, (T, H))
    sign = rng.choice([-1.0, 1.0], (T, H))
    x = workloads.to_bf16_bits((sign * mant * np.exp2(expo.astype(np.float64))).astype(np.float32))
    x[3, ::7] = 0x8000  # -0.0
    x[4, ::5] = 0x0000
    x[5] = workloads.to_bf16_bits(rng.standard_normal(H) * 1e-30)  # a row of tiny values only
    wr = workloads.to_bf16_bits(rng.standard_normal((8, H)) / 64)
    check_route(x, wr, None, 2, tag="many binades")



@pytest.mark.parametrize("T,H,E,k", [
    (5, 8192, 8, 2),    # rows past 4096 values: four waves per token
    (3, 6144, 8, 2),    # 12 chunks per lane: the 16-chunk kernel with four chunks past the row
    (7, 4096, 16, 4),   # sixteen experts: two per wave of the eight-wave kernel
    (2, 4096, 3, 2),    # fewer experts than waves
])
def test_route_small_batches_wave_split(T, H, E, k):
    """The small-batch launch shape (one workgroup per token, the experts split over its
    waves, the top-k and the quantisation in separate waves): ids, logits, codes and
    scales bit-exact, with a bias."""
    rng = np.random.default_rng(T * 131 + H + E)
    x = workloads.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = workloads.to_bf16_bits((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    bias = rng.standard_normal(E).astype(np.float32) * 0.1
    check_route(x, wr, bias, k, tag=f"small batch E={E}")
