"""Pins of the oracle's expert math: closed forms, brute-force dense-then-mask,
the full softmax mixture, exact scaling. References here use numpy float64
matrix products and torch's bf16/e4m3fn casts (library routines), never the
oracle's own code."""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import workloads


def _bf16_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def _fp8_f64(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def _to_fp8_codes(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).clamp(-448, 448).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e8m0_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e8m0fnu).double().numpy()


def _mx_quant(a):
    """MX block quantisation along the last axis from numpy's log2 and torch's casts."""
    R, C = a.shape
    b = a.astype(np.float64).reshape(R, C // 32, 32)
    amax = np.abs(b).max(2)
    x = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0)
    x = np.clip(x, -127, 127)
    codes = _to_fp8_codes((b * np.exp2(-x)[:, :, None]).reshape(R, C))
    return _fp8_f64(codes) * np.exp2(x).repeat(32, axis=1)


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0,
                  -4.0, -6.0])  # the OCP E2M1 values by code


def _fp4_f64(packed):
    """Packed E2M1 codes (value 2i in the low nibble of byte i) -> values by table lookup."""
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(*packed.shape[:-1], -1)
    return _E2M1[codes]


def deq_weights(inp):
    if inp.wl.dtype == "mxfp4":
        return tuple(_fp4_f64(w) * _e8m0_f64(s).repeat(32, axis=2)
                     for w, s in ((inp.w1, inp.s1), (inp.w3, inp.s3), (inp.w2, inp.s2)))
    if inp.wl.dtype == "bf16":
        return _bf16_f64(inp.w1), _bf16_f64(inp.w3), _bf16_f64(inp.w2)
    if inp.wl.dtype == "mxfp8":
        return tuple(_fp8_f64(w) * _e8m0_f64(s).repeat(32, axis=2)
                     for w, s in ((inp.w1, inp.s1), (inp.w3, inp.s3), (inp.w2, inp.s2)))
    return (_fp8_f64(inp.w1) * inp.s1[:, :, None], _fp8_f64(inp.w3) * inp.s3[:, :, None],
            _fp8_f64(inp.w2) * inp.s2[:, :, None])


def token_inputs(inp):
    x = _bf16_f64(inp.x)
    if inp.wl.dtype == "bf16":
        return x
    if inp.wl.dtype in ("mxfp8", "mxfp4"):
        return _mx_quant(x)
    xf = x.astype(np.float32)
    amax = np.abs(xf).max(1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = _to_fp8_codes(xf / s[:, None])
    return _fp8_f64(q) * s[:, None].astype(np.float64)


def store(dtype, a):
    if dtype == "bf16":
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
    if dtype in ("mxfp8", "mxfp4"):  # bf16 storage, then the MXFP8 block quantisation
        return _mx_quant(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy())
    amax = np.abs(a).max(1, keepdims=True)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    return _fp8_f64(_to_fp8_codes((a / s).astype(np.float32))) * s


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_outputs(inp, xh):
    """Every expert applied to every token: Y[e, t, :] (dense, no routing)."""
    W1, W3, W2 = deq_weights(inp)
    Y = []
    for e in range(inp.wl.E):
        a = silu(xh @ W1[e].T) * (xh @ W3[e].T)
        Y.append(store(inp.wl.dtype, a) @ W2[e].T)
    return np.stack(Y)


def rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


def small(dtype, E, k, T=24, H=256, I=384, seed=9, bias=None):
    wl = workloads.Workload("t", T, H, I, E, k, dtype, 1.0, 1.0 / np.sqrt(H), 0.05, seed)
    inp = workloads.generate(wl)
    if bias is not None:
        inp.bias = np.asarray(bias, np.float32)
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8", "mxfp4"])
def test_single_expert_equals_swiglu_mlp(dtype):
    inp = small(dtype, E=1, k=1)
    out, o64 = oracle.forward(inp)
    xh = token_inputs(inp)
    ref = expert_outputs(inp, xh)[0]
    assert rel(o64, ref) < 1e-9
    ref_b = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.mean(out.view(np.int16) == ref_b) > 0.999


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8", "mxfp4"])
def test_dense_then_mask_equals_routed(dtype):
    wl = workloads.config(0)
    if dtype != "bf16":
        wl = workloads.scaled(wl, dtype=dtype)
    inp = workloads.generate(wl)
    out, o64 = oracle.forward(inp)
    ids, w, _ = oracle.route(inp.x, inp.w_router, None, wl.k)
    Y = expert_outputs(inp, token_inputs(inp))
    mask = np.zeros((wl.T, wl.E))
    for t in range(wl.T):
        for j in range(wl.k):
            mask[t, ids[t, j]] = w[t, j]
    ref = np.einsum("te,eth->th", mask, Y)
    assert rel(o64, ref) < 1e-9


def test_k_equal_E_is_full_softmax_mixture():
    inp = small("bf16", E=4, k=4)
    _, o64 = oracle.forward(inp)
    _, _, lg = oracle.route(inp.x, inp.w_router, None, 4)
    p = softmax(lg.astype(np.float64), axis=1)
    Y = expert_outputs(inp, token_inputs(inp))
    ref = np.einsum("te,eth->th", p, Y)
    assert rel(o64, ref) < 1e-6  # routing weights are fp32


def test_bias_pair_routing():
    inp = small("fp8", E=8, k=2, bias=[0, 0, 0, 60.0, 0, 0, 0, 90.0])
    _, o64 = oracle.forward(inp)
    ids, w, lg = oracle.route(inp.x, inp.w_router, inp.bias, 2)
    assert np.all(ids == [7, 3])
    Y = expert_outputs(inp, token_inputs(inp))
    ref = w[:, :1] * Y[7] + w[:, 1:] * Y[3]
    assert rel(o64, ref) < 1e-9


def test_doubling_down_weights_doubles_output_exactly():
    inp = small("bf16", E=4, k=2)
    _, o64 = oracle.forward(inp)
    w2 = inp.w2.copy()
    w2 = (w2.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1 (no zeros/subnormals here)
    assert np.all((inp.w2 & 0x7F80) != 0)
    inp.w2 = w2
    _, o64b = oracle.forward(inp)
    assert np.array_equal(o64b, 2.0 * o64)


@pytest.mark.parametrize("dtype", ["mxfp8", "mxfp4"])
def test_mx_down_scale_code_plus_one_doubles_output_exactly(dtype):
    inp = small(dtype, E=4, k=2)
    _, o64 = oracle.forward(inp)
    assert np.all(inp.s2 < 254)
    inp.s2 = (inp.s2 + 1).astype(np.uint8)
    _, o64b = oracle.forward(inp)
    assert np.array_equal(o64b, 2.0 * o64)


def test_mx_gate_scale_block_is_used_per_32_columns():
    # raising the scale code of one 32-column block of W1 changes the result exactly as
    # doubling those 32 weight values does in the dense reference
    inp = small("mxfp8", E=1, k=1)
    inp.s1 = inp.s1.copy()
    inp.s1[0, :, 3] += 1
    _, o64 = oracle.forward(inp)
    ref = expert_outputs(inp, token_inputs(inp))[0]
    assert rel(o64, ref) < 1e-9
    inp2 = small("mxfp8", E=1, k=1)
    _, o64_0 = oracle.forward(inp2)
    assert rel(o64, o64_0) > 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8", "mxfp4"])
def test_swiglu_and_down_rows(dtype):
    inp = small(dtype, E=4, k=2)
    xh = token_inputs(inp)
    W1, W3, W2 = deq_weights(inp)
    tokens = np.array([0, 5, 5, 23], np.int32)
    experts = np.array([3, 0, 1, 3], np.int32)
    a = oracle.swiglu(dtype, inp.x, inp.w1, inp.w3, inp.s1, inp.s3, tokens, experts)
    ref = np.stack([silu(xh[t] @ W1[e].T) * (xh[t] @ W3[e].T) for t, e in zip(tokens, experts)])
    assert rel(a, ref) < 1e-12
    st = oracle.store_intermediate(dtype, a)
    assert rel(st, store(dtype, ref)) < 1e-12
    y = oracle.down(dtype, st, inp.w2, inp.s2, experts)
    yref = np.stack([st[r] @ W2[e].T for r, e in enumerate(experts)])
    assert rel(y, yref) < 1e-12
