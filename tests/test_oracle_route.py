"""Pins of the oracle's router (logits, top-k, renormalised weights) and of the
per-token fp8 activation quantisation."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(a):
    return workloads.to_bf16_bits(np.asarray(a, np.float32))


def f(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def test_canonical_summation_order_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "canonical_logit.json")))
    H = g["H"]
    x = np.zeros(H, np.float32)
    w = np.zeros(H, np.float32)
    for h, xv, wv in g["nonzero"]:
        x[h], w[h] = xv, wv
    got = oracle.logit(bf16(x), bf16(w))
    assert float(got) == g["expected_logit"]
    assert g["expected_logit"] not in g["other_orders"].values()


def test_logits_within_fp32_bound_of_exact_dot():
    wl = workloads.config(0)
    inp = workloads.generate(wl, weights=False)
    _, _, lg = oracle.route(inp.x, inp.w_router, None, wl.k)
    X, W = f(inp.x), f(inp.w_router)
    exact = X @ W.T
    depth = wl.H // 64 + 6  # sequential adds per partial + folding levels
    u = 2.0 ** -24
    bound = depth * u / (1 - depth * u) * (np.abs(X) @ np.abs(W).T)
    assert np.all(np.abs(lg.astype(np.float64) - exact) <= bound)


def test_topk_matches_bruteforce_sort():
    wl = workloads.config(0)
    inp = workloads.generate(wl, weights=False)
    for k in (1, 2, 3, 8):
        ids, w, lg = oracle.route(inp.x, inp.w_router, None, k)
        for t in range(wl.T):
            order = sorted(range(wl.E), key=lambda e: (-float(lg[t, e]), e))
            assert list(ids[t]) == order[:k]
            sel = lg[t, order[:k]].astype(np.float64)
            np.testing.assert_allclose(w[t], softmax(sel), rtol=2e-7, atol=0)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * 2.0 ** -23)


def test_k_equal_one_weight_is_one():
    wl = workloads.config(0)
    inp = workloads.generate(wl, weights=False)
    _, w, _ = oracle.route(inp.x, inp.w_router, None, 1)
    assert np.all(w == 1.0)


def test_ties_go_to_lower_index():
    H, E = 128, 8
    rng = np.random.default_rng(11)
    wr = bf16(rng.standard_normal((E, H)) / np.sqrt(H))
    wr[5] = wr[3]
    x = bf16(rng.standard_normal((64, H)))
    ids, w, lg = oracle.route(x, wr, None, E)
    assert np.array_equal(lg[:, 3], lg[:, 5])
    for t in range(64):
        r = list(ids[t])
        assert r.index(3) < r.index(5)
        assert w[t, r.index(3)] == w[t, r.index(5)]


def test_zero_token_all_logits_zero():
    H, E = 128, 8
    x = np.zeros((2, H), np.uint16)
    x[1] = 0x8000  # -0.0 everywhere
    wr = bf16(np.random.default_rng(1).standard_normal((E, H)))
    ids, w, lg = oracle.route(x, wr, None, 2)
    assert np.all(lg == 0.0)
    assert ids.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == 0.5)
    ids, w, _ = oracle.route(x, wr, None, 4)
    assert np.all(w == 0.25)


def test_bias_forces_experts_and_enters_weights():
    wl = workloads.config(0)
    inp = workloads.generate(wl, weights=False)
    bias = np.zeros(wl.E, np.float32)
    bias[6], bias[2] = 100.0, 50.0
    ids, w, lg = oracle.route(inp.x, inp.w_router, bias, 2)
    assert np.all(ids == np.array([6, 2]))
    _, _, lg0 = oracle.route(inp.x, inp.w_router, None, 2)
    assert np.array_equal(lg, (lg0 + bias).astype(np.float32))
    np.testing.assert_allclose(w, softmax(lg[:, [6, 2]].astype(np.float64), axis=1), rtol=2e-7)


def test_topk_of_given_logits_equals_route():
    wl = workloads.config(0)
    inp = workloads.generate(wl, weights=False)
    ids, w, lg = oracle.route(inp.x, inp.w_router, None, 2)
    ids2, w2 = oracle.topk(lg, 2)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)


def test_token_quantisation_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = bf16(rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1))))
    x[3] = 0
    q, s = oracle.quant_tokens(x)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    amax = xt.abs().amax(1)
    st = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    assert np.array_equal(s, st.numpy())
    qt = (xt / st[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, qt)
    # every non-zero row reaches the top code; dequantised error within half a step
    mag = q & 0x7F
    assert np.all(mag[np.arange(64) != 3].max(1) == 0x7E)
    deq = oracle.e4m3fn_to_f64(q) * s[:, None].astype(np.float64)
    err = np.abs(deq - xt.double().numpy())
    assert np.all(err <= np.maximum(np.abs(xt.double().numpy()) * 2.0 ** -4, 2.0 ** -10 * s[:, None]))
