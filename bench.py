"""Benchmark of the routed top-k MoE layer on one MI355X.

One step = one whole layer call (route + FP8 token quantisation, align, stage 1,
stage 2 with requantisation and combine) on the Mixtral 8x7B expert shape in
FP8 e4m3fn at T=8192 tokens (H=4096, I=14336, E=8, top-2), inputs resident in
HBM, weights preshuffled once before timing. Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload prefill|decode16]
                    [--no-cpu-baseline] [--cpu-tokens 24]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5000.0, "bf16": 2500.0}  # dense MFMA TFLOP/s, MI355X published
HBM_PEAK = 8000.0                       # GB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pick_workload(name):
    import workloads
    if name == "prefill":
        return workloads.config(2)
    if name == "decode16":
        return workloads.config(3, 16)
    if name == "bf16-decode":
        return workloads.config(1)
    if name == "skewed":
        return workloads.config(4)
    raise SystemExit(f"unknown workload {name}")


def cpu_baseline(inp, n_tokens):
    """The CPU oracle, as it stands, on the first n_tokens tokens of the same workload."""
    import oracle
    wl = inp.wl
    toks = np.arange(min(n_tokens, wl.T), dtype=np.int32)
    t0 = time.perf_counter()
    oracle.forward(inp, toks)
    dt = time.perf_counter() - t0
    flops = 6.0 * wl.H * wl.I * wl.k * toks.size
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"whole layer (route, quantise, {wl.k} experts, combine) for the first "
                      f"{toks.size} tokens of {wl.name}: {dt:.1f} s wall, effective flops "
                      f"6*H*I per token-slot"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=24)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer is built and timed on a single "
              f"MI355X (got --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        raise SystemExit(2)

    import torch
    import workloads
    import mixture_experts_routed_top_amd as moe

    wl = pick_workload(args.workload)
    log(f"[bench] generating {wl.name}")
    inp = workloads.generate(wl, threads=16)
    dev = lambda a: None if a is None else torch.from_numpy(
        np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else np.ascontiguousarray(a)
    ).to("cuda")
    x, wr, bias = dev(inp.x), dev(inp.w_router), dev(inp.bias)
    w1, w3, w2 = dev(inp.w1), dev(inp.w3), dev(inp.w2)
    layer = moe.Layer(wl.dtype, wr, w1, w3, w2, dev(inp.s1), dev(inp.s3), dev(inp.s2), bias,
                      wl.k, wl.T)
    del w1, w3, w2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] block_m={layer.bm}; warmup {args.warmup}")

    for _ in range(args.warmup):
        layer(x)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        layer(x, events=ev[i])
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    s1_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    log(f"[bench] {ms:.3f} ms/step, stage-1 kernel {s1_ms:.3f} ms")

    flops = wl.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    s1_flops = 4.0 * wl.H * wl.I * wl.slots  # gate + up GEMMs: 2 * 2*H*I per slot
    s1_tf = s1_flops / (s1_ms * 1e-3) / 1e12
    peak = PEAK[wl.dtype]
    traffic_path = os.path.join(ROOT, "profiles", "stage1_traffic.json")
    traffic = None
    if os.path.exists(traffic_path):
        with open(traffic_path) as f:
            t = json.load(f)
        if t.get("workload") == wl.name and t.get("kernel_source_sha") == _kernel_sha():
            traffic = t.get("bytes_per_launch")

    rec = {
        "metric": "MoE layer effective TFLOP/s + tokens/s, Mixtral 8x7B shape, FP8, T=16..8192",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3fn (fp32 accumulate, bf16 out)" if wl.dtype == "fp8" else "bf16",
        "data": "synthetic (seeded normals, Mixtral 8x7B expert shapes; no trained weights)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
                   "block_m": layer.bm, "frac_of_fp8_peak_whole_layer": round(tflops / peak, 4)},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel stage 1 (gate/up + SwiGLU)",
                     "achieved": round(s1_tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(s1_tf / peak, 4), "traffic": traffic,
                     "avg_launch_ms": round(s1_ms, 4)},
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(rec), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_routed_top_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
