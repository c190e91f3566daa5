"""Benchmark of the routed top-k MoE layer on one MI355X.

One step = one whole layer call (route + FP8 token quantisation, align, stage 1,
stage 2 with requantisation and combine) on the Mixtral 8x7B expert shape in
FP8 e4m3fn at T=8192 tokens (H=4096, I=14336, E=8, top-2), inputs resident in
HBM, weights preshuffled once before timing. Prints one JSON line whose value
is the effective TFLOP/s of the whole layer (6*H*I flops per token-slot).

The same line carries:
  roofline      stage-1 kernel (gather + gate/up GEMM + SwiGLU, the dominant
                kernel) against the FP8 matrix-core peak, its launch time taken
                with HIP events on the stream it runs on; traffic = HBM bytes
                per launch from the committed counter summary (null if the
                kernel source changed since);
  decode_sweep  the FP8 decode batches T = 1, 4, 16, 64, 256: median latency of
                100 single calls (HIP events around each call; a 512 MB buffer is
                read before each call, untimed, so the Infinity Cache holds no
                weights from the previous one), tokens/s, and weight-read
                bandwidth over the active experts' weight bytes against 8 TB/s;
  bf16_decode   the same for the BF16 decode batch T=16;
  skewed        the FP8 skewed workload (T=16384, ~40% of slots on expert 0):
                latency, effective TFLOP/s, slots and row tiles per expert, pad rows;
  mxfp8         the MXFP8 layer (E8M0 scale per 32 values): prefill T=8192 (whole
                layer and stage-1 kernel TFLOP/s) and the decode batch T=16 measured
                like the FP8 sweep;
  mxfp4         the layer with MXFP4 (E2M1) expert weights and MXFP8 tokens: prefill
                T=8192 and the decode sweep T = 1 .. 256, weight GB/s over the
                active experts' codes and scales;
  backward      the bf16 layer's backward pass (moe_backward) at the Mixtral shape and
                T=8192: ms per call and TFLOP/s (12*H*I flops per token-slot), with
                the bf16 forward on the same batch timed beside it;
  cpu_baseline  the CPU oracle on the first tokens of the same workload; per_workload
                holds its wall time (oracle_s, cores) on up to 16 tokens of each of the
                other workloads (the tiny layer, the BF16 decode batch, each FP8 decode
                batch and the skewed layer).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-sweep]
                    [--no-cpu-baseline] [--cpu-tokens 64] [--copy-calibration]
                    [--decode-runs 100]
    python bench.py --decode-only T [--decode-runs N]   (one FP8 decode batch)
    python bench.py --mxfp8-only [--steps K]           (the MXFP8 lines only)
    python bench.py --mxfp4-only [--steps K]           (the MXFP4 lines only)
    python bench.py --backward-only [--steps K]        (the bf16 backward line only)
    python bench.py --traffic-from FETCH.db WRITE.db   (writes the traffic summary)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5000.0, "bf16": 2500.0}  # dense matrix-core TFLOP/s, MI355X published
HBM_PEAK = 8000.0                       # GB/s, MI355X published
TRAFFIC = os.path.join(ROOT, "profiles", "stage1_traffic.json")
METRIC = "MoE layer effective TFLOP/s + tokens/s, Mixtral 8x7B shape, FP8, T=16..8192"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    """Hash of the sources the stage-1 kernel is compiled from (the GEMM file and the two
    headers it includes): a traffic figure is only valid for the code it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_routed_top_amd", "csrc")
    for n in ("gemm.hip", "moe_device.h", "moe_launch.h"):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def make_layer(inp, block_m=None):
    import mixture_experts_routed_top_amd as moe
    wl = inp.wl
    w1, w3, w2 = dev(inp.w1), dev(inp.w3), dev(inp.w2)
    layer = moe.Layer(wl.dtype, dev(inp.w_router), w1, w3, w2, dev(inp.s1), dev(inp.s3),
                      dev(inp.s2), dev(inp.bias), wl.k, wl.T, block_m)
    del w1, w3, w2  # only the preshuffled copies stay resident
    return layer


def cpu_baseline(inp, n_tokens):
    """The CPU oracle, as it stands, on the first n_tokens tokens of the same workload."""
    wl = inp.wl
    r = oracle_time(inp, n_tokens)
    return {"value": r["tflops"], "unit": "TFLOP/s", "cores": r["cores"], "kind": "oracle",
            "sample": f"whole layer (route, quantise, {wl.k} experts, combine) for the first "
                      f"{r['tokens']} of {wl.T} tokens of {wl.name}: {r['oracle_s']:.1f} s wall; "
                      f"effective flops 6*H*I per token-slot"}


ORACLE_TIMES = []  # one record per workload, filled by the legs that have its inputs


def oracle_time(inp, n_tokens):
    """Wall time of the CPU oracle (whole layer) on the first n_tokens tokens of a workload
    (all of them when the batch is smaller), recorded in ORACLE_TIMES."""
    import oracle
    wl = inp.wl
    toks = np.arange(min(n_tokens, wl.T), dtype=np.int32)
    t0 = time.perf_counter()
    oracle.forward(inp, toks)
    dt = time.perf_counter() - t0
    rec = {"workload": wl.name, "T": wl.T, "tokens": int(toks.size), "oracle_s": round(dt, 3),
           "oracle_s_per_token": round(dt / toks.size, 4), "cores": oracle.threads(),
           "tflops": round(6.0 * wl.H * wl.I * wl.k * toks.size / dt / 1e12, 6)}
    ORACLE_TIMES.append(rec)
    log(f"[bench] oracle {wl.name}: {toks.size} tokens in {dt:.2f} s")
    return rec


def evict(flush):
    """Read the whole flush buffer (a reduction, untimed), so that the 256 MB Infinity Cache
    holds none of the weights of the previous call. A read leaves no dirty lines: a buffer
    rewritten here instead would leave up to the cache's size of dirty data, whose write-back
    to HBM then runs during the timed call (measured: about 40 us more per call at every
    decode batch size, the same for reading the buffer after rewriting it)."""
    return flush.sum()


def timed_calls(layer, x, runs, flush):
    """Median and mean latency (ms) of `runs` single layer calls, each bracketed by HIP
    events on the current stream, with the flush buffer read (untimed) before each call."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(runs)]
    for i in range(runs):
        evict(flush)
        ev[i][0].record()
        layer(x)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return float(np.median(ms)), float(ms.mean())


def decode_line(wl, layer, x, runs, flush, bytes_per_weight):
    import torch
    for _ in range(5):
        layer(x)
    torch.cuda.synchronize()
    med, mean = timed_calls(layer, x, runs, flush)
    active = int(torch.unique(layer.ids).numel())
    wbytes = active * 3 * wl.H * wl.I * bytes_per_weight  # weights of the experts that get a slot
    gbps = wbytes / (med * 1e-3) / 1e9
    log(f"[bench] {wl.name}: median {med * 1e3:.1f} us, {gbps:.0f} GB/s over {active} experts")
    return {"T": wl.T, "ms": round(med, 4), "ms_mean": round(mean, 4),
            "tokens_per_s": round(wl.T / (med * 1e-3), 1), "active_experts": active,
            "weight_gbps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK, 4),
            "tflops": round(wl.flops() / (med * 1e-3) / 1e12, 2)}


def calibration_copy():
    """One 1 GiB device-to-device copy: the reference reading for the byte counters."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def flush_buffer():
    import torch
    return torch.zeros(128 << 20, dtype=torch.float32, device="cuda")  # 512 MB, 2x the Infinity Cache


def decode_sweep(runs, oracle_tokens=0):
    """FP8 decode batches: per-T median latency of the whole layer over `runs` calls with
    the Infinity Cache flushed between calls, tokens/s, weight GB/s (and, with
    oracle_tokens, the CPU oracle's time on up to that many tokens of each batch)."""
    import torch
    import workloads
    base = workloads.generate(workloads.config(3, workloads.DECODE_SWEEP[0]), threads=16)
    layer = make_layer(base)
    flush = flush_buffer()
    torch.cuda.synchronize()
    out = []
    for T in workloads.DECODE_SWEEP:
        wl = workloads.config(3, T)
        xi = workloads.generate(wl, weights=False)
        x = dev(xi.x)
        out.append(decode_line(wl, layer, x, runs, flush, 1))
        if oracle_tokens:
            oracle_time(workloads.Inputs(wl, xi.x, base.w_router, None, base.w1, base.w3, base.w2,
                                         base.s1, base.s3, base.s2), oracle_tokens)
    del layer, flush
    torch.cuda.empty_cache()
    return out


def bf16_decode(runs, oracle_tokens=0):
    """The BF16 decode batch (Mixtral shape, T=16), measured like the FP8 sweep."""
    import torch
    import workloads
    wl = workloads.config(1)
    inp = workloads.generate(wl, threads=16)
    layer = make_layer(inp)
    flush = flush_buffer()
    rec = decode_line(wl, layer, dev(inp.x), runs, flush, 2)
    if oracle_tokens:
        oracle_time(inp, oracle_tokens)
    rec = {"workload": wl.name, **rec}
    del layer, flush
    torch.cuda.empty_cache()
    return rec


def skewed(steps, oracle_tokens=0):
    """The skewed FP8 workload (T=16384, ~40% of slots on expert 0): latency, effective
    TFLOP/s, and what the skew does to the grouping (slots and row tiles per expert, pad rows)."""
    import torch
    import workloads
    wl = workloads.config(4)
    inp = workloads.generate(wl, threads=16)
    layer = make_layer(inp)
    x = dev(inp.x)
    for _ in range(3):
        layer(x)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        layer(x)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    count = layer.grp.count.cpu().numpy().astype(int)
    total = int(layer.grp.total.cpu().numpy()[0])
    bm = layer.bm
    tiles = [int(-(-c // bm)) for c in count]
    tf = wl.flops() / (ms * 1e-3) / 1e12
    log(f"[bench] {wl.name}: {ms:.3f} ms, {tf:.0f} TFLOP/s, expert slots {count.tolist()}")
    del layer
    torch.cuda.empty_cache()
    if oracle_tokens:
        oracle_time(inp, oracle_tokens)
    return {"workload": wl.name, "T": wl.T, "ms": round(ms, 4), "tflops": round(tf, 2),
            "frac_of_fp8_peak": round(tf / PEAK["fp8"], 4),
            "tokens_per_s": round(wl.T / (ms * 1e-3), 1), "block_m": bm,
            "expert_slots": count.tolist(),
            "expert_share": [round(c / wl.slots, 4) for c in count],
            "expert_row_tiles": tiles, "padded_rows": total,
            "pad_fraction": round((total - wl.slots) / total, 4)}


def backward_line(steps, T=8192):
    """The bf16 layer's backward pass (moe_backward: gradients of x, W1, W3, W2, the router
    weights and the router bias, the top-k selection held fixed) at the Mixtral shape on a
    prefill batch of T tokens, with the forward timed beside it. Weights and router are the
    bf16 decode workload's (seed 1), x its generator's draw for T tokens, dout seeded normals.
    TFLOP/s count 6*H*I flops per token-slot for the forward and 12*H*I for the backward.
    The forward is the training one (it keeps the pre-activations g, u) and the backward
    uses them; backward_recompute_ms is the backward that recomputes them instead."""
    import torch
    import mixture_experts_routed_top_amd as moe
    import workloads
    wl = workloads.scaled(workloads.config(1), name=f"mixtral-bf16-T{T}", T=T)
    log(f"[bench] generating {wl.name} (backward)")
    inp = workloads.generate(wl, threads=16)
    w1, w3, w2 = dev(inp.w1), dev(inp.w3), dev(inp.w2)
    layer = moe.Layer("bf16", dev(inp.w_router), w1, w3, w2, None, None, None, None, wl.k, T,
                      save_preact=True)
    w2t, w13t = moe.preshuffle_backward(w1, w3, w2)
    del w1, w3, w2
    x = dev(inp.x)
    dout = dev(workloads.to_bf16_bits(
        np.random.default_rng(7).standard_normal((T, wl.H)).astype(np.float32)))

    def bw(gu=layer.gu):
        return moe.backward(x, layer.w_router, layer.ids, layer.w, layer.grp, layer.act,
                            layer.pw, w2t, w13t, dout, gu=gu)

    layer(x)
    for _ in range(2):
        g = bw()
    torch.cuda.synchronize()
    del g
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        layer(x)
    t1.record()
    torch.cuda.synchronize()
    fwd = t0.elapsed_time(t1) / steps
    t0.record()
    for _ in range(steps):
        bw()
    t1.record()
    torch.cuda.synchronize()
    bwd = t0.elapsed_time(t1) / steps
    t0.record()
    for _ in range(steps):
        bw(None)
    t1.record()
    torch.cuda.synchronize()
    bwd_rc = t0.elapsed_time(t1) / steps
    fl = wl.flops()
    log(f"[bench] {wl.name}: forward {fwd:.3f} ms, backward {bwd:.3f} ms "
        f"({bwd_rc:.3f} ms recomputing the pre-activations)")
    out = {"workload": wl.name, "T": T, "block_m": layer.bm,
           "forward_ms": round(fwd, 4), "forward_tflops": round(fl / (fwd * 1e-3) / 1e12, 2),
           "backward_ms": round(bwd, 4),
           "backward_tflops": round(2 * fl / (bwd * 1e-3) / 1e12, 2),
           "backward_frac_of_bf16_peak": round(2 * fl / (bwd * 1e-3) / 1e12 / PEAK["bf16"], 4),
           "backward_recompute_ms": round(bwd_rc, 4),
           "tokens_per_s_forward_backward": round(T / ((fwd + bwd) * 1e-3), 1)}
    del layer, w2t, w13t, x, dout
    torch.cuda.empty_cache()
    return out


def timed_steps(layer, x, steps):
    """Mean whole-layer ms over `steps` back-to-back calls and the mean stage-1 kernel ms
    (HIP events on the stream the stages run on)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        layer(x, events=ev[i])
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def mx_lines(kind, steps, runs, decode_ts):
    """A block-scaled layer ("mxfp8" or "mxfp4") at the Mixtral shape: prefill T=8192
    (whole layer and stage-1 kernel) and the decode batches decode_ts, measured like the
    FP8 sweep over the active experts' weight bytes (codes plus one E8M0 byte per 32)."""
    import torch
    import workloads
    make_wl = getattr(workloads, kind)
    wl = make_wl(8192)
    inp = workloads.generate(wl, threads=16)
    layer = make_layer(inp)
    x = dev(inp.x)
    for _ in range(3):
        layer(x)
    ms, s1_ms = timed_steps(layer, x, steps)
    tf = wl.flops() / (ms * 1e-3) / 1e12
    s1_tf = 4.0 * wl.H * wl.I * wl.slots / (s1_ms * 1e-3) / 1e12
    log(f"[bench] {wl.name}: {ms:.3f} ms, {tf:.0f} TFLOP/s; stage 1 {s1_ms:.3f} ms")
    prefill = {"workload": wl.name, "T": wl.T, "block_m": layer.bm, "ms": round(ms, 4),
               "tflops": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK["fp8"], 4),
               "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
               "stage1_ms": round(s1_ms, 4), "stage1_tflops": round(s1_tf, 2),
               "stage1_frac": round(s1_tf / PEAK["fp8"], 4)}
    flush = flush_buffer()
    per_weight = (0.5 if kind == "mxfp4" else 1.0) + 1.0 / 32.0
    dec = []
    for T in decode_ts:
        wd = make_wl(T)
        rec = decode_line(wd, layer, dev(workloads.generate(wd, weights=False).x), runs, flush,
                          per_weight)
        dec.append({"workload": wd.name, **rec})
    del layer, flush
    torch.cuda.empty_cache()
    return {"prefill": prefill, "decode": dec[0] if len(dec) == 1 else dec}


def mxfp8(steps, runs):
    """The MXFP8 layer: prefill T=8192 and decode T=16."""
    return mx_lines("mxfp8", steps, runs, (16,))


def mxfp4(steps, runs):
    """The MXFP4-weight layer: prefill T=8192 and the decode sweep T = 1 .. 256."""
    import workloads
    return mx_lines("mxfp4", steps, runs, workloads.DECODE_SWEEP)


def traffic_from(fetch_db, write_db):
    """Stage-1 HBM bytes per launch from two rocprofv3 --pmc databases (FETCH_SIZE,
    WRITE_SIZE, in KiB per dispatch), each scaled by the same counter's reading for the
    1 GiB device copy that --copy-calibration runs in the same program."""
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, value from counters_collection "
                           "where counter_name=?", (counter,)).fetchall()
        s1 = [v for n, v in rows if "gemm_kernel<1, 1," in n]
        copy = [v for n, v in rows if "copyBuffer" in n and v > 500000]
        if not s1 or not copy:
            raise SystemExit(f"{db}: no stage-1 or calibration-copy dispatch with {counter}")
        return float(np.mean(s1)), float(max(copy))

    f_s1, f_copy = per_kernel(fetch_db, "FETCH_SIZE")
    w_s1, w_copy = per_kernel(write_db, "WRITE_SIZE")
    kib = float(1 << 20)  # the calibration copy reads and writes 1 GiB = 2^20 KiB
    f_scale, w_scale = kib / f_copy, kib / w_copy
    rec = {"workload": "mixtral-fp8-prefill-T8192", "kernel": "stage 1 (gemm_kernel<1, 1, ...>)",
           "kernel_source_sha": kernel_sha(),
           "fetch_kib_raw": round(f_s1, 1), "write_kib_raw": round(w_s1, 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "bytes_per_launch": int((f_s1 * f_scale + w_s1 * w_scale) * 1024)}
    with open(TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--decode-runs", type=int, default=100,
                    help="single calls per decode batch (median reported)")
    ap.add_argument("--decode-only", type=int, metavar="T", default=None,
                    help="only time the FP8 decode batch T (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--oracle-tokens", type=int, default=16,
                    help="tokens of each other workload the CPU oracle is timed on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--mxfp8-only", action="store_true",
                    help="only the MXFP8 prefill and decode lines (for profiler runs)")
    ap.add_argument("--mxfp4-only", action="store_true",
                    help="only the MXFP4 prefill and decode lines (for profiler runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the bf16 backward line at T=8192 (for profiler runs)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer is built and timed on a single "
              f"MI355X (got --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        raise SystemExit(2)

    import torch
    import workloads

    if args.mxfp8_only:
        print(json.dumps({"mxfp8": mxfp8(args.steps, args.decode_runs)}), flush=True)
        return
    if args.mxfp4_only:
        print(json.dumps({"mxfp4": mxfp4(args.steps, args.decode_runs)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": backward_line(args.steps)}), flush=True)
        return

    if args.decode_only is not None:
        wl = workloads.config(3, args.decode_only)
        inp = workloads.generate(wl, threads=16)
        layer = make_layer(inp)
        print(json.dumps({"decode": decode_line(wl, layer, dev(inp.x), args.decode_runs,
                                                flush_buffer(), 1)}), flush=True)
        if args.copy_calibration:
            calibration_copy()
        return

    wl = workloads.config(2)
    log(f"[bench] generating {wl.name}")
    inp = workloads.generate(wl, threads=16)
    layer = make_layer(inp, args.block_m)
    x = dev(inp.x)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] block_m={layer.bm}; warmup {args.warmup}")
    for _ in range(args.warmup):
        layer(x)
    torch.cuda.synchronize()

    # Timed region: K whole-layer steps; stage 1 bracketed by events on the same stream.
    ms, s1_ms = timed_steps(layer, x, args.steps)
    log(f"[bench] {ms:.3f} ms/step, stage-1 kernel {s1_ms:.3f} ms")

    tflops = wl.flops() / (ms * 1e-3) / 1e12
    s1_flops = 4.0 * wl.H * wl.I * wl.slots  # gate + up GEMMs: 2 * 2*H*I per token-slot
    s1_tf = s1_flops / (s1_ms * 1e-3) / 1e12
    peak = PEAK[wl.dtype]
    traffic = None
    if os.path.exists(TRAFFIC):
        with open(TRAFFIC) as f:
            t = json.load(f)
        if t.get("workload") == wl.name and t.get("kernel_source_sha") == kernel_sha():
            traffic = t.get("bytes_per_launch")

    if args.copy_calibration:
        calibration_copy()
    del layer
    torch.cuda.empty_cache()

    rec = {
        "metric": METRIC,
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
        "dtype": "fp8_e4m3fn",
        "data": "synthetic (seeded normals, Mixtral 8x7B expert shapes; no trained weights)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
                   "block_m": args.block_m or __import__(
                       "mixture_experts_routed_top_amd").pick_block_m(wl.T, wl.k, wl.E),
                   "accumulate": "fp32", "output": "bf16",
                   "frac_of_fp8_peak_whole_layer": round(tflops / peak, 4)},
        "roofline": {"bound": "mfma", "kernel": "stage 1: gather + gate/up FP8 GEMM + SwiGLU",
                     "achieved": round(s1_tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(s1_tf / peak, 4), "traffic": traffic,
                     "avg_launch_ms": round(s1_ms, 4)},
    }
    ot = 0 if args.no_cpu_baseline else args.oracle_tokens
    if not args.no_sweep:
        rec["decode_sweep"] = decode_sweep(args.decode_runs, ot)
        rec["bf16_decode"] = bf16_decode(args.decode_runs, ot)
        rec["skewed"] = skewed(max(5, args.steps // 2), ot)
        rec["mxfp8"] = mxfp8(max(5, args.steps // 2), args.decode_runs)
        rec["mxfp4"] = mxfp4(max(5, args.steps // 2), args.decode_runs)
        rec["backward"] = backward_line(max(5, args.steps // 2))
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
        oracle_time(workloads.generate(workloads.config(0)), 32)
        rec["cpu_baseline"]["per_workload"] = ORACLE_TIMES
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
