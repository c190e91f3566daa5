"""Pins of the oracle's backward pass (the bf16 layer's gradients with the top-k
selection held fixed).

- torch.autograd in float64 on a dense "every expert, then mask" formulation of
  the layer written here (a library routine differentiating an independent
  expression of the same function);
- central finite differences of the oracle's fp64 forward along random
  directions of every parameter (and of x);
- invariants: the routing weights sum to 1 for every parameter value, so the
  selected logits' gradients sum to zero per token (the bias gradient sums to
  zero); experts that receive no slot get zero weight gradients; doubling dout
  doubles every gradient exactly.
References never call the oracle's backward code."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _bf16_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double()


def make(T, H, I, E, k, seed, bias=False):
    wl = workloads.Workload(f"bwd-{T}-{H}-{I}-{E}-{k}", T, H, I, E, k, "bf16", 1.0,
                            1.0 / np.sqrt(H), 0.2, seed)
    inp = workloads.generate(wl)
    if bias:
        inp.bias = np.linspace(-0.5, 0.5, E).astype(np.float32)
    rng = np.random.default_rng(seed + 100)
    dout = workloads.to_bf16_bits(rng.standard_normal((T, H)))
    return inp, dout


def autograd_reference(inp, dout, ids):
    """Gradients by torch.autograd (float64) of sum <dout, out> with
    out_t = sum_e mask_te * softmax_selected(l_t)_e * W2_e (silu(W1_e x_t) * W3_e x_t),
    every expert computed densely and masked with the given selection."""
    x = _bf16_f64(inp.x).requires_grad_()
    wr = _bf16_f64(inp.w_router).requires_grad_()
    w1 = _bf16_f64(inp.w1).requires_grad_()
    w3 = _bf16_f64(inp.w3).requires_grad_()
    w2 = _bf16_f64(inp.w2).requires_grad_()
    b = torch.zeros(inp.wl.E, dtype=torch.float64) if inp.bias is None else \
        torch.from_numpy(inp.bias.astype(np.float64))
    b.requires_grad_()
    E = inp.wl.E
    mask = torch.zeros(x.shape[0], E, dtype=torch.bool)
    mask[torch.arange(x.shape[0])[:, None], torch.from_numpy(ids.astype(np.int64))] = True
    logits = x @ wr.T + b                                          # [T, E]
    p = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=1)  # 0 off the selection
    g = torch.einsum("eih,th->tei", w1, x)
    u = torch.einsum("eih,th->tei", w3, x)
    a = torch.nn.functional.silu(g) * u                            # [T, E, I]
    y = torch.einsum("ehi,tei->teh", w2, a)                        # [T, E, H]
    out = (p[:, :, None] * y).sum(1)
    loss = (out * _bf16_f64(dout)).sum()
    loss.backward()
    return dict(dx=x.grad.numpy(), dw1=w1.grad.numpy(), dw3=w3.grad.numpy(),
                dw2=w2.grad.numpy(), dw_router=wr.grad.numpy(), dbias=b.grad.numpy())


CASES = [
    (6, 32, 48, 4, 2, 0, False),
    (5, 64, 32, 8, 8, 1, True),    # k = E: the full softmax mixture, with a bias
    (4, 32, 32, 1, 1, 2, False),   # E = 1, k = 1: a plain SwiGLU MLP (router gradient 0)
    (9, 64, 64, 8, 2, 3, True),
]


@pytest.mark.parametrize("T,H,I,E,k,seed,bias", CASES)
def test_backward_matches_autograd_of_dense_masked_layer(T, H, I, E, k, seed, bias):
    inp, dout = make(T, H, I, E, k, seed, bias)
    ids, _, _ = oracle.route(inp.x, inp.w_router, inp.bias, k)
    got = oracle.backward(inp, dout)
    ref = autograd_reference(inp, dout, ids)
    for name in ("dx", "dw1", "dw3", "dw2", "dw_router", "dbias"):
        r, o = ref[name], got[name]
        scale = max(np.abs(r).max(), 1e-300)
        assert np.abs(o - r).max() <= 1e-11 * scale + 1e-300, name


def _f64_params(inp):
    f = lambda a: _bf16_f64(a).numpy()
    b = None if inp.bias is None else inp.bias.astype(np.float64)
    return dict(x=f(inp.x), wr=f(inp.w_router), w1=f(inp.w1), w3=f(inp.w3), w2=f(inp.w2), b=b)


@pytest.mark.parametrize("T,H,I,E,k,seed,bias", CASES[:2] + CASES[3:])
def test_backward_matches_finite_differences(T, H, I, E, k, seed, bias):
    inp, dout = make(T, H, I, E, k, seed, bias)
    ids, _, _ = oracle.route(inp.x, inp.w_router, inp.bias, k)
    got = oracle.backward(inp, dout)
    P = _f64_params(inp)
    d = _bf16_f64(dout).numpy()
    rng = np.random.default_rng(seed + 7)

    def loss(Q):
        out = oracle.forward_f64(Q["x"], Q["wr"], Q["b"], Q["w1"], Q["w3"], Q["w2"], ids)
        return float((out * d).sum())

    grads = dict(x="dx", wr="dw_router", w1="dw1", w3="dw3", w2="dw2", b="dbias")
    for key, gname in grads.items():
        if P[key] is None:
            continue
        V = rng.standard_normal(P[key].shape)
        eps = 1e-6 * np.abs(P[key]).max() / np.abs(V).max()
        plus = dict(P); plus[key] = P[key] + eps * V
        minus = dict(P); minus[key] = P[key] - eps * V
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float((got[gname] * V).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), abs(fd), 1e-12), (key, fd, an)


def test_backward_invariants():
    T, H, I, E, k = 12, 64, 48, 8, 2
    inp, dout = make(T, H, I, E, k, 5, bias=True)
    # route every token to experts 0..5 only: experts 6 and 7 get no slot
    inp.bias = np.array([0, 0, 0, 0, 0, 0, -1e4, -1e4], np.float32)
    ids, _, _ = oracle.route(inp.x, inp.w_router, inp.bias, k)
    assert not np.isin(ids, [6, 7]).any()
    g = oracle.backward(inp, dout)
    for name in ("dw1", "dw3", "dw2", "dw_router"):
        assert not g[name][6:].any(), name
    assert g["dbias"][6:].sum() == 0.0
    # the selected logits' gradients sum to zero per token, so the bias gradient does
    assert abs(g["dbias"].sum()) <= 1e-12 * np.abs(g["dbias"]).max()
    # the gradients are linear in dout: doubling it (exact in bf16) doubles each exactly
    d2 = workloads.to_bf16_bits(2.0 * _bf16_f64(dout).numpy().astype(np.float32))
    g2 = oracle.backward(inp, d2)
    for name in g:
        assert np.array_equal(g2[name], 2.0 * g[name]), name


def test_forward_f64_agrees_with_the_layer_oracle():
    """The fp64 forward the gradients differentiate is the layer the oracle computes, up to
    the bf16 storage of the intermediate that oracle.forward applies."""
    inp, _ = make(8, 64, 96, 8, 2, 9)
    ids, _, _ = oracle.route(inp.x, inp.w_router, None, 2)
    P = _f64_params(inp)
    exact = oracle.forward_f64(P["x"], P["wr"], None, P["w1"], P["w3"], P["w2"], ids)
    _, o64 = oracle.forward(inp)
    assert np.abs(exact - o64).max() <= 1e-2 * np.abs(exact).max()
