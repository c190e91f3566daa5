"""The seeded workloads: determinism, shapes, and the skewed workload's routing shares."""
import numpy as np

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
