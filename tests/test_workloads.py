"""The seeded workloads: determinism, shapes, and the skewed workload's routing shares."""
import numpy as np
import torch

import oracle
import workloads


def test_generation_is_deterministic():
    wl = workloads.config(0)
    a, b = workloads.generate(wl), workloads.generate(wl)
    for n in ("x", "w_router", "w1", "w3", "w2"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    assert a.x.shape == (32, 128) and a.w1.shape == (8, 256, 128) and a.w2.shape == (8, 128, 256)


def test_fp8_weights_use_per_channel_amax_scale():
    wl = workloads.scaled(workloads.config(0), dtype="fp8")
    inp = workloads.generate(wl)
    # every output channel reaches the top code 448 (scale = amax/448)
    assert np.all((inp.w1 & 0x7F).max(2) == 0x7E)
    assert np.all((inp.w2 & 0x7F).max(2) == 0x7E)
    assert inp.s1.shape == (8, 256) and inp.s2.shape == (8, 128)


def test_skewed_workload_shares():
    wl = workloads.config(4)
    inp = workloads.generate(wl, weights=False)
    ids, _, _ = oracle.route(inp.x, inp.w_router, inp.bias, wl.k)
    share = np.bincount(ids.ravel(), minlength=wl.E) / ids.size
    assert 0.39 <= share[0] <= 0.41
    assert share[6] < 0.03 and share[7] < 0.03


def test_mx_weight_blocks_dequantise_to_the_drawn_values():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    q, s = workloads.quantize_blocks_mx(a)
    assert q.shape == a.shape and s.shape == (64, 8) and s.dtype == np.uint8
    vals = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    deq = vals * torch.from_numpy(s).view(torch.float8_e8m0fnu).double().numpy().repeat(32, 1)
    scale = torch.from_numpy(s).view(torch.float8_e8m0fnu).double().numpy().repeat(32, 1)
    err = np.abs(deq - a) / np.abs(a).reshape(64, 8, 32).max(2).repeat(32, 1)
    sat = np.abs(a) / scale > 448
    assert err[~sat].max() <= 2.0 ** -4  # at most half an ulp of the block's top binade
    assert np.all(np.abs(deq[sat]) == 448 * scale[sat])
    assert workloads.mxfp8(16).dtype == "mxfp8" and workloads.mxfp8(16).H == 4096
