"""Seeded synthetic inputs for the routed top-k MoE layer.

This module only draws random numbers and stores them in the input formats the
layer consumes (bf16 bit patterns, OCP e4m3fn codes with per-channel fp32
scales). It holds none of the layer's own arithmetic: no routing, no top-k, no
GEMM, no SwiGLU, no activation quantisation. Both the CPU oracle and the HIP
path take their inputs from here, so they see identical bytes.

Five workloads: a tiny bf16 layer, and the Mixtral 8x7B expert layer (H=4096, I=14336, E=8,
top-2) in bf16 decode, fp8 prefill, an fp8 decode sweep and an fp8 layer with
skewed routing. Mixtral 8x7B in FP8 is the model the first page (the FlyDSL-in-JAX
talk summary, "Wichtigste Punkte", 5:56-9:14) measures on; the pages use no dataset.

Weight quantisation for the fp8 workloads (one fp32 scale per output channel,
scale = amax/448, codes by round-to-nearest-even with saturation) is load-time
input preparation, done here with torch's float8_e4m3fn cast. It is not part of
the hot path: the library's entry points take the codes and scales as inputs.
The MXFP8 workloads (the second page, the PyTorch FlyDSL backend news item,
"Grenzen und Folgen für Anwender": E4M3 values with one E8M0 scale per 32 along
the reduction; its "Gemessene Leistung" measurements start from quantised
operands) store the weights the same way per 32-value block of each row, with
the OCP MX scale 2^(floor(log2 amax) - 8). The MXFP4 workloads (the packed E2M1
operands of the same section) store E2M1 weight codes, two per byte, with the
scale 2^(floor(log2 amax) - 2) (6 = 1.5 * 2^2 is E2M1's largest value).
"""
from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

MIXTRAL = dict(H=4096, I=14336, E=8, k=2)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str            # "bf16", "fp8", "mxfp8" or "mxfp4" (weights; tokens mxfp8)
    sigma_x: float
    sigma_r: float
    sigma_w: float
    seed: int
    skewed: bool = False  # router bias that sends ~40% of slots to expert 0
    x_seed: tuple = field(default=())  # extra seed words for x only (decode sweep)

    @property
    def slots(self) -> int:
        return self.T * self.k

    def flops(self) -> float:
        """Useful flops of one layer call: 2*3*H*I per token-slot."""
        return 6.0 * self.H * self.I * self.slots


def config(i: int, T: int | None = None) -> Workload:
    """The i-th workload (0..4). Workload 3 is a sweep; pass T in {1,4,16,64,256}."""
    m = MIXTRAL
    if i == 0:
        return Workload("tiny-bf16-T32", 32, 128, 256, 8, 2, "bf16",
                        1.0, 1.0 / math.sqrt(128.0), 0.05, 0)
    if i == 1:
        return Workload("mixtral-bf16-decode-T16", 16, m["H"], m["I"], m["E"], m["k"], "bf16",
                        1.0, 1.0 / 64.0, 0.02, 1)
    if i == 2:
        return Workload("mixtral-fp8-prefill-T8192", 8192, m["H"], m["I"], m["E"], m["k"], "fp8",
                        1.0, 1.0 / 64.0, 0.02, 2)
    if i == 3:
        T = 16 if T is None else int(T)
        assert T in DECODE_SWEEP, T
        return Workload(f"mixtral-fp8-decode-T{T}", T, m["H"], m["I"], m["E"], m["k"], "fp8",
                        1.0, 1.0 / 64.0, 0.02, 3, x_seed=(T,))
    if i == 4:
        return Workload("mixtral-fp8-skewed-T16384", 16384, m["H"], m["I"], m["E"], m["k"], "fp8",
                        1.0, 1.0 / 64.0, 0.02, 4, skewed=True)
    raise ValueError(i)


DECODE_SWEEP = (1, 4, 16, 64, 256)


def mxfp4(T: int) -> Workload:
    """The Mixtral expert layer with MXFP4 expert weights (and MXFP8 tokens) at batch T;
    weights and router drawn like the fp8 workloads, seed 6."""
    m = MIXTRAL
    return Workload(f"mixtral-mxfp4-T{T}", int(T), m["H"], m["I"], m["E"], m["k"], "mxfp4",
                    1.0, 1.0 / 64.0, 0.02, 6, x_seed=(int(T),))


def mxfp8(T: int) -> Workload:
    """The Mixtral expert layer with MXFP8 operands (block-scaled weights and tokens) at
    batch T; weights and router drawn like the fp8 workloads, seed 5."""
    m = MIXTRAL
    return Workload(f"mixtral-mxfp8-T{T}", int(T), m["H"], m["I"], m["E"], m["k"], "mxfp8",
                    1.0, 1.0 / 64.0, 0.02, 5, x_seed=(int(T),))


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (used for small parity shapes)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# ---------------------------------------------------------------------------
# format helpers (storage only)

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (torch's round-to-nearest-even cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_rows_fp8(a: np.ndarray):
    """Per-row (output channel) e4m3fn codes and fp32 scales, scale = amax/448.

    Returns (codes uint8 [R, C], scales float32 [R]). A row of zeros gets scale 1.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    amax = t.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / s[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), s.numpy().astype(np.float32)


def quantize_blocks_mx(a: np.ndarray, block: int = 32):
    """Per-block e4m3fn codes and E8M0 scale codes along each row (OCP MX storage).

    Block b of row r (columns b*block .. +block-1) gets exponent
    x = floor(log2 amax) - 8 (0 for an all-zero block), clamped to [-127, 127];
    codes = e4m3fn(clamp(a / 2^x, -448, 448)). Returns (codes uint8 [R, C],
    scale codes uint8 [R, C/block] = x + 127).
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    R, C = t.shape
    b = t.reshape(R, C // block, block)
    amax = b.abs().amax(dim=2)
    _, ex = torch.frexp(amax)  # amax = m * 2^ex with 0.5 <= m < 1
    x = torch.where(amax > 0, (ex - 9).clamp(-127, 127), torch.zeros_like(ex))
    q = torch.ldexp(b, (-x).unsqueeze(2).to(torch.float32)).clamp(-448.0, 448.0)
    q = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return q.numpy(), (x + 127).to(torch.uint8).numpy()


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)  # between E2M1 values


def quantize_blocks_mx4(a: np.ndarray, block: int = 32):
    """Per-block E2M1 codes (packed two per byte, value 2i in the low nibble of byte i)
    and E8M0 scale codes along each row (OCP MX storage).

    Block b of row r gets exponent x = floor(log2 amax) - 2 (0 for an all-zero block),
    clamped to [-127, 127]; codes = nearest E2M1 value of clamp(a / 2^x, -6, 6), ties to
    the even code (E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are codes 0..7). Returns
    (codes uint8 [R, C/2], scale codes uint8 [R, C/block])."""
    a = np.ascontiguousarray(a, np.float32)
    R, C = a.shape
    b = a.reshape(R, C // block, block)
    amax = np.abs(b).max(2)
    _, ex = np.frexp(amax)  # amax = m * 2^ex, 0.5 <= m < 1
    x = np.where(amax > 0, np.clip(ex - 3, -127, 127), 0)
    v = np.clip(b * np.exp2(-x).astype(np.float32)[:, :, None], -6.0, 6.0).reshape(R, C)
    mag = np.abs(v)
    code = np.searchsorted(_E2M1_MID, mag, side="left")  # midpoints below |v|
    tie = (code < 7) & (mag == _E2M1_MID[np.minimum(code, 6)])
    code = (code + (tie & (code % 2 == 1))).astype(np.uint8)  # a tie goes to the even code
    code |= np.signbit(v).astype(np.uint8) << 3
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (x + 127).astype(np.uint8)


# ---------------------------------------------------------------------------

@dataclass
class Inputs:
    """Host copies of one workload's inputs, in the layer's storage formats."""
    wl: Workload
    x: np.ndarray            # uint16 bf16 [T, H]
    w_router: np.ndarray     # uint16 bf16 [E, H]
    bias: np.ndarray | None  # float32 [E] or None
    w1: np.ndarray           # bf16 uint16 or e4m3fn uint8 [E, I, H] (gate); mxfp4 [E, I, H/2]
    w3: np.ndarray           # same, [E, I, H] (up)
    w2: np.ndarray           # same, [E, H, I] (down); mxfp4 [E, H, I/2]
    s1: np.ndarray | None    # fp8: float32 [E, I]; mxfp8: E8M0 uint8 [E, I, H/32]
    s3: np.ndarray | None    # same as s1
    s2: np.ndarray | None    # fp8: float32 [E, H]; mxfp8: E8M0 uint8 [E, H, I/32]


def _normal(seed_words, shape, sigma) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(list(seed_words)))
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def skew_bias(E: int) -> np.ndarray:
    """Router bias of the skewed workload: (beta, 0, ..., 0, -gamma, -gamma).

    beta and gamma were calibrated once by workloads/calibrate_skew.py (which
    routes with the oracle) and stored in skew_bias.json.
    """
    with open(os.path.join(_HERE, "skew_bias.json")) as f:
        d = json.load(f)
    b = np.zeros(E, np.float32)
    b[0] = d["beta"]
    b[E - 2] = -d["gamma"]
    b[E - 1] = -d["gamma"]
    return b


def generate(wl: Workload, weights: bool = True, threads: int = 8) -> Inputs:
    """Draw the inputs of a workload. Tensors are drawn in the fixed order
    x, W_r, W1, W3, W2 from independent child streams of the workload's seed."""
    T, H, I, E = wl.T, wl.H, wl.I, wl.E
    x = to_bf16_bits(_normal((wl.seed, 0) + tuple(wl.x_seed), (T, H), wl.sigma_x))
    wr = to_bf16_bits(_normal((wl.seed, 1), (E, H), wl.sigma_r))
    bias = skew_bias(E) if wl.skewed else None
    if not weights:
        return Inputs(wl, x, wr, bias, None, None, None, None, None, None)

    # One child stream per (matrix, expert) so experts can be drawn in parallel.
    jobs = []
    for m, (rows, cols) in enumerate(((I, H), (I, H), (H, I))):
        for e in range(E):
            jobs.append((m, e, rows, cols))

    def draw(job):
        m, e, rows, cols = job
        a = _normal((wl.seed, 2 + m, e), (rows, cols), wl.sigma_w)
        if wl.dtype == "bf16":
            return job, to_bf16_bits(a), None
        if wl.dtype == "mxfp8":
            q, s = quantize_blocks_mx(a)
            return job, q, s
        if wl.dtype == "mxfp4":
            q, s = quantize_blocks_mx4(a)
            return job, q, s
        q, s = quantize_rows_fp8(a)
        return job, q, s

    wdt = np.uint16 if wl.dtype == "bf16" else np.uint8
    per = 2 if wl.dtype == "mxfp4" else 1  # values per stored element
    w1 = np.empty((E, I, H // per), wdt)
    w3 = np.empty((E, I, H // per), wdt)
    w2 = np.empty((E, H, I // per), wdt)
    mats = (w1, w3, w2)
    fp8 = wl.dtype in ("fp8", "mxfp8", "mxfp4")
    if wl.dtype in ("mxfp8", "mxfp4"):
        s1 = np.empty((E, I, H // 32), np.uint8)
        s3 = np.empty((E, I, H // 32), np.uint8)
        s2 = np.empty((E, H, I // 32), np.uint8)
    else:
        s1 = np.empty((E, I), np.float32) if fp8 else None
        s3 = np.empty((E, I), np.float32) if fp8 else None
        s2 = np.empty((E, H), np.float32) if fp8 else None
    scales = (s1, s3, s2)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for (m, e, _, _), q, s in ex.map(draw, jobs):
            mats[m][e] = q
            if fp8:
                scales[m][e] = s
    return Inputs(wl, x, wr, bias, w1, w3, w2, s1, s3, s2)
