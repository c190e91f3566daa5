"""Calibrate the router bias of the skewed Mixtral fp8 workload (T=16384).

The skewed workload uses a per-expert router bias under which expert 0 receives
about 40% of the token-slots and experts 6 and 7 under 3% each. With bias
b = (beta, 0, 0, 0, 0, 0, -gamma, -gamma), this script routes the workload's
seeded tokens with the CPU oracle and bisects gamma (shares of experts 6 and 7
near 2%) and beta (share of expert 0 near 40%), then writes skew_bias.json.

Run once: python -m workloads.calibrate_skew
"""
import json
import os

import numpy as np

import oracle
import workloads

TARGET0 = 0.40
TARGET_TAIL = 0.02


def shares(inp, beta, gamma):
    E = inp.wl.E
    b = np.zeros(E, np.float32)
    b[0], b[E - 2], b[E - 1] = beta, -gamma, -gamma
    ids, _, _ = oracle.route(inp.x, inp.w_router, b, inp.wl.k)
    return np.bincount(ids.ravel(), minlength=E) / ids.size


def bisect(fn, lo, hi, target, increasing, iters=30):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        v = fn(mid)
        if (v < target) == increasing:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main():
    wl = workloads.scaled(workloads.config(4), skewed=False)  # unbiased draws of x and W_r
    inp = workloads.generate(wl, weights=False)
    beta, gamma = 0.0, 0.0
    for _ in range(3):
        gamma = bisect(lambda g: max(shares(inp, beta, g)[6:]), 0.0, 8.0, TARGET_TAIL, False)
        beta = bisect(lambda b: shares(inp, b, gamma)[0], 0.0, 8.0, TARGET0, True)
    beta, gamma = float(np.float32(beta)), float(np.float32(gamma))
    s = shares(inp, beta, gamma)
    assert 0.39 <= s[0] <= 0.41 and max(s[6:]) < 0.03, s
    out = dict(beta=beta, gamma=gamma, shares=[round(float(v), 5) for v in s],
               note="router bias (beta,0,0,0,0,0,-gamma,-gamma) of the skewed fp8 workload; "
                    "written by workloads/calibrate_skew.py using the CPU oracle's router")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
