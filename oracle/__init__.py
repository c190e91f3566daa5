"""CPU oracle of the routed top-k MoE layer (ctypes front end of moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. The product path never imports this package.

Every function takes numpy arrays in the layer's storage formats (bf16 as
uint16 bit patterns, e4m3fn as uint8 codes) and returns numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")

BF16, FP8, MXFP8, MXFP4 = 0, 1, 2, 3


def build() -> str:
    """Compile moe_oracle.c with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", LIB_PATH + ".tmp", SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        L.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f32_to_e4m3fn.restype = ctypes.c_uint8
        L.oracle_f32_to_e4m3fn.argtypes = [ctypes.c_float]
        L.oracle_logit.restype = ctypes.c_float
        L.oracle_logit.argtypes = [P, P, i]
        L.oracle_route.argtypes = [P, P, P, i, i, i, i, P, P, P]
        L.oracle_topk.argtypes = [P, i, i, i, P, P]
        L.oracle_quant_tokens.argtypes = [P, i, i, P, P]
        L.oracle_quant_tokens_mx.argtypes = [P, i, i, P, P]
        L.oracle_e8m0_to_f64.restype = ctypes.c_double
        L.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_align.restype = ctypes.c_int
        L.oracle_align.argtypes = [P, i, i, i, i, P, P, P, P, P]
        L.oracle_swiglu.argtypes = [i, P, P, P, P, P, i, i, i, P, P, i, P]
        L.oracle_down.argtypes = [i, P, P, P, i, i, P, i, P]
        L.oracle_forward.argtypes = [i, P, P, P, P, P, P, P, P, P, i, i, i, i, i, P, i, P, P]
        L.oracle_store_intermediate.argtypes = [i, P, i, i]
        L.oracle_preshuffle_w13.argtypes = [i, i, i, i, P, P, P]
        L.oracle_preshuffle_w2.argtypes = [i, i, i, i, P, P]
        L.oracle_forward_f64.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P]
        L.oracle_backward.argtypes = [P, P, P, P, P, P, i, i, i, i, i, P, P, P, P, P, P, P]
        L.oracle_threads.restype = ctypes.c_int
        for name in ("oracle_f32_to_e4m3fn_n", "oracle_e4m3fn_to_f64_n",
                     "oracle_f32_to_bf16_n", "oracle_bf16_to_f64_n", "oracle_e8m0_to_f64_n",
                     "oracle_e2m1_to_f64_n", "oracle_f32_to_e2m1_n"):
            getattr(L, name).argtypes = [P, ctypes.c_long, P]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(dtype: str) -> int:
    return {"bf16": BF16, "fp8": FP8, "mxfp8": MXFP8, "mxfp4": MXFP4}[dtype]


# --- number formats --------------------------------------------------------

def _conv(fn, a, in_dt, out_dt):
    a = np.ascontiguousarray(a, in_dt)
    out = np.empty(a.shape, out_dt)
    fn(_p(a), ctypes.c_long(a.size), _p(out))
    return out


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_bf16_to_f64_n, b, np.uint16, np.float64)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_f32_to_bf16_n, f, np.float32, np.uint16)


def e4m3fn_to_f64(q: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_e4m3fn_to_f64_n, q, np.uint8, np.float64)


def f32_to_e4m3fn(f: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_f32_to_e4m3fn_n, f, np.float32, np.uint8)


def e8m0_to_f64(b: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_e8m0_to_f64_n, b, np.uint8, np.float64)


def e2m1_to_f64(q: np.ndarray) -> np.ndarray:
    """E2M1 codes (low 4 bits of each byte) -> values."""
    return _conv(lib().oracle_e2m1_to_f64_n, q, np.uint8, np.float64)


def f32_to_e2m1(f: np.ndarray) -> np.ndarray:
    return _conv(lib().oracle_f32_to_e2m1_n, f, np.float32, np.uint8)


# --- router ----------------------------------------------------------------

def logit(x_row: np.ndarray, w_row: np.ndarray) -> np.float32:
    x_row = np.ascontiguousarray(x_row, np.uint16)
    w_row = np.ascontiguousarray(w_row, np.uint16)
    return np.float32(lib().oracle_logit(_p(x_row), _p(w_row), x_row.size))


def route(x, w_router, bias, k):
    """-> (ids int32 [T,k], weights float32 [T,k], logits float32 [T,E])."""
    x = np.ascontiguousarray(x, np.uint16)
    w_router = np.ascontiguousarray(w_router, np.uint16)
    T, H = x.shape
    E = w_router.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lg = np.empty((T, E), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().oracle_route(_p(x), _p(w_router), _p(b), T, H, E, k, _p(ids), _p(w), _p(lg))
    return ids, w, lg


def topk(logits, k):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().oracle_topk(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def quant_tokens(x):
    """-> (codes uint8 [T,H], scales float32 [T])."""
    x = np.ascontiguousarray(x, np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty((T,), np.float32)
    lib().oracle_quant_tokens(_p(x), T, H, _p(q), _p(s))
    return q, s


def quant_tokens_mx(x):
    """MX block quantisation of token rows -> (codes uint8 [T,H], E8M0 codes uint8 [T,H/32])."""
    x = np.ascontiguousarray(x, np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 32), np.uint8)
    lib().oracle_quant_tokens_mx(_p(x), T, H, _p(q), _p(s))
    return q, s


# --- grouping --------------------------------------------------------------

def capacity(T, k, E, bm):
    """Rows that any grouping of T*k slots over E experts can need after padding."""
    return -(-(T * k + E * (bm - 1)) // bm) * bm


def align(ids, E, bm):
    """-> dict(sorted_slot, tile_expert, count, offset, total) (prefix [0,total) valid)."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    cap = capacity(T, k, E, bm)
    ss = np.full(cap, -1, np.int32)
    te = np.full(cap // bm, -1, np.int32)
    cnt = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    tot = np.empty(1, np.int32)
    rc = lib().oracle_align(_p(ids), T, k, E, bm, _p(ss), _p(te), _p(cnt), _p(off), _p(tot))
    if rc != 0:
        raise ValueError("expert id out of range")
    n = int(tot[0])
    return dict(sorted_slot=ss[:n], tile_expert=te[: n // bm], count=cnt, offset=off, total=n)


# --- expert math -----------------------------------------------------------

def swiglu(dtype, x, w1, w3, s1, s3, tokens, experts):
    """SwiGLU intermediate (before storage rounding), fp64 [n, I]."""
    x = np.ascontiguousarray(x, np.uint16)
    T, H = x.shape
    I = w1.shape[1]
    tokens = np.ascontiguousarray(tokens, np.int32)
    experts = np.ascontiguousarray(experts, np.int32)
    out = np.empty((tokens.size, I), np.float64)
    lib().oracle_swiglu(_dt(dtype), _p(x), _p(w1), _p(w3), _p(s1), _p(s3), T, H, I,
                        _p(tokens), _p(experts), tokens.size, _p(out))
    return out


def store_intermediate(dtype, act):
    """Storage rounding of the intermediate (bf16; per-row e4m3fn requantisation; or bf16
    followed by the MX block quantisation)."""
    a = np.array(act, np.float64, copy=True, order="C")
    lib().oracle_store_intermediate(_dt(dtype), _p(a), a.shape[0], a.shape[1])
    return a


def down(dtype, act, w2, s2, experts):
    """Down projection of intermediate rows act[n, I] (fp64 values) -> fp64 [n, H]."""
    act = np.ascontiguousarray(act, np.float64)
    experts = np.ascontiguousarray(experts, np.int32)
    H, I = w2.shape[1], act.shape[1]  # w2 rows hold I values (I/2 bytes for packed E2M1)
    y = np.empty((experts.size, H), np.float64)
    lib().oracle_down(_dt(dtype), _p(act), _p(w2), _p(s2), H, I, _p(experts), experts.size, _p(y))
    return y


def forward(inp, tokens=None):
    """Whole layer for the listed tokens of a workloads.Inputs.

    -> (out bf16 uint16 [n, H], out before the final rounding fp64 [n, H])."""
    wl = inp.wl
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, np.int32)
    n = tokens.size
    out = np.empty((n, wl.H), np.uint16)
    o64 = np.empty((n, wl.H), np.float64)
    lib().oracle_forward(_dt(wl.dtype), _p(inp.x), _p(inp.w_router), _p(inp.bias),
                         _p(inp.w1), _p(inp.w3), _p(inp.w2), _p(inp.s1), _p(inp.s3), _p(inp.s2),
                         wl.T, wl.H, wl.I, wl.E, wl.k, _p(tokens), n, _p(out), _p(o64))
    return out, o64


# --- backward pass (bf16 layer) -------------------------------------------

def forward_f64(x, w_router, bias, w1, w3, w2, ids):
    """fp64 layer output for fp64 parameters and a fixed selection ids [T,k] (no storage
    roundings): the function whose gradients backward() returns."""
    x, w_router, w1, w3, w2 = (np.ascontiguousarray(a, np.float64)
                               for a in (x, w_router, w1, w3, w2))
    b = None if bias is None else np.ascontiguousarray(bias, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    T, H = x.shape
    E, I = w1.shape[0], w1.shape[1]
    out = np.empty((T, H), np.float64)
    lib().oracle_forward_f64(_p(x), _p(w_router), _p(b), _p(w1), _p(w3), _p(w2), _p(ids), T, H,
                             I, E, ids.shape[1], _p(out))
    return out


def backward(inp, dout):
    """Gradients of sum <dout, out> for a bf16 workloads.Inputs and a bf16 dout [T,H]:
    dict(dx [T,H], dw1 [E,I,H], dw3 [E,I,H], dw2 [E,H,I], dw_router [E,H], dbias [E]),
    all fp64, the selection held at the forward's."""
    wl = inp.wl
    assert wl.dtype == "bf16", "the backward is defined for the bf16 layer"
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    dout = np.ascontiguousarray(dout, np.uint16)
    r = dict(dx=np.empty((T, H)), dw1=np.empty((E, I, H)), dw3=np.empty((E, I, H)),
             dw2=np.empty((E, H, I)), dw_router=np.empty((E, H)), dbias=np.empty(E))
    b = None if inp.bias is None else np.ascontiguousarray(inp.bias, np.float32)
    lib().oracle_backward(_p(inp.x), _p(inp.w_router), _p(b), _p(inp.w1), _p(inp.w3),
                          _p(inp.w2), T, H, I, E, k, _p(dout), _p(r["dx"]), _p(r["dw1"]),
                          _p(r["dw3"]), _p(r["dw2"]), _p(r["dw_router"]), _p(r["dbias"]))
    return r


# --- preshuffle layout -----------------------------------------------------

def preshuffle(dtype, w1, w3, w2):
    """Weights in the GPU library's MFMA-operand order (a byte relayout)."""
    E, I, H = w1.shape
    w13p = np.empty(2 * w1.size * w1.itemsize, np.uint8)
    w2p = np.empty(w2.size * w2.itemsize, np.uint8)
    L = lib()
    L.oracle_preshuffle_w13(_dt(dtype), E, H, I, _p(np.ascontiguousarray(w1)),
                            _p(np.ascontiguousarray(w3)), _p(w13p))
    L.oracle_preshuffle_w2(_dt(dtype), E, H, I, _p(np.ascontiguousarray(w2)), _p(w2p))
    return w13p, w2p


def threads() -> int:
    return int(lib().oracle_threads())
