"""Helpers of the GPU parity tests: upload workloads, run the library, compare."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

import mixture_experts_routed_top_amd as moe

TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp8": 5e-2, "mxfp4": 5e-2}  # max|err| / max|ref| of the layer output


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray | None) -> torch.Tensor | None:
    """Host array (bf16 as uint16, e4m3fn as uint8, fp32, int32) -> device tensor, same bytes."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


class Uploaded:
    """A workload's inputs on the device plus its preshuffled layer."""

    def __init__(self, inp, block_m=None):
        self.inp = inp
        wl = inp.wl
        self.x = dev(inp.x)
        self.wr = dev(inp.w_router)
        self.bias = dev(inp.bias)
        w1, w3, w2 = dev(inp.w1), dev(inp.w3), dev(inp.w2)
        s1, s3, s2 = dev(inp.s1), dev(inp.s3), dev(inp.s2)
        self.layer = moe.Layer(wl.dtype, self.wr, w1, w3, w2, s1, s3, s2, self.bias, wl.k, wl.T,
                               block_m)
        del w1, w3, w2

    def run(self) -> np.ndarray:
        out = self.layer(self.x)
        torch.cuda.synchronize()
        return host(out)


def rel_err(out_bf16: np.ndarray, ref_f64: np.ndarray) -> float:
    return float(np.abs(bf16_to_f64(out_bf16) - ref_f64).max() / np.abs(ref_f64).max())


def sample_tokens(ids: np.ndarray, E: int, n: int, seed: int = 0) -> np.ndarray:
    """n tokens spread over the batch, covering every expert that has a slot, the first
    and the last token."""
    T = ids.shape[0]
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    for e in range(E):
        hit = np.nonzero((ids == e).any(1))[0]
        if hit.size:
            pick.add(int(hit[rng.integers(hit.size)]))
    rest = [t for t in rng.permutation(T) if t not in pick]
    pick.update(int(t) for t in rest[: max(0, n - len(pick))])
    return np.array(sorted(pick), np.int32)


def tile_rows(block_m: int) -> int:
    """Rows of one GEMM row tile for a grouping with M-tile block_m (both stages tile the
    grouped rows in 32-, 64- or 128-row tiles that never straddle two experts)."""
    return min(block_m, 128)


def cover_tokens(ids: np.ndarray, E: int, block_m: int, seed: int = 0) -> np.ndarray:
    """Tokens whose layer outputs, compared element by element, touch every live row tile of
    both GEMM stages: one real slot drawn from each row tile of the grouping (a slot's output
    row spans every feature tile of stage 2, and its intermediate row every feature tile of
    stage 1), plus the first and the last token. The grouping is the oracle's."""
    import oracle
    T, k = ids.shape
    g = oracle.align(ids, E, block_m)
    ss, tr = g["sorted_slot"], tile_rows(block_m)
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    for r0 in range(0, g["total"], tr):
        real = ss[r0:r0 + tr]
        real = real[real < T * k]
        if real.size:
            pick.add(int(real[rng.integers(real.size)]) // k)
    return np.array(sorted(pick), np.int32)


def live_row_tiles(ids: np.ndarray, E: int, block_m: int) -> int:
    import oracle
    return oracle.align(ids, E, block_m)["total"] // tile_rows(block_m)


ERROR_LOG = os.environ.get("MOE_PARITY_LOG", os.path.join(
    os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
    "parity_errors.jsonl"))


def record_error(case: str, err: float, tol: float, tokens: int, total_tokens: int, **extra):
    """Append one parity figure (max|err|/max|ref| of the layer output) to the JSONL log."""
    rec = {"case": case, "rel_err": err, "tolerance": tol, "tokens_checked": tokens,
           "tokens": total_tokens, "time": time.strftime("%Y-%m-%d %H:%M:%S"), **extra}
    try:
        os.makedirs(os.path.dirname(ERROR_LOG), exist_ok=True)
        with open(ERROR_LOG, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError as e:  # a read-only tree must not fail the parity test itself
        say(f"(parity log not written: {e})")
