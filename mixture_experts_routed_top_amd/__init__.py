"""Routed top-k mixture-of-experts layer for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of libmoe.so (include/moe.h): it allocates the
outputs as torch tensors on the current device, passes raw device pointers and
the current HIP stream, and checks status codes. All computation happens in the
library's HIP kernels; torch provides device memory and streams only.

    ids, w, x_q, x_scale, _ = route(x, w_router, k, fp8=True)
    grp = align(ids, E, block_m)
    pw = preshuffle("fp8", w1, w3, w2, s1, s3, s2)          # once, at load time
    act, amax = stage1("fp8", x_q, x_scale, pw, grp)
    out = stage2("fp8", act, amax, pw, grp, w)

The MXFP8 path ("mxfp8": e4m3fn values with one E8M0 scale code per 32 values
along the reduction) is the same sequence with route(..., mx=True), which
returns the block codes of x as x_scale, and block-scaled weights. The MXFP4
path ("mxfp4") takes packed E2M1 expert weights (two per byte, [E, I, H/2] and
[E, H, I/2]) with the same E8M0 block codes; tokens are MXFP8 as before.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from ._lib import BF16, FP8, MXFP4, MXFP8, MoEError, check, lib

__all__ = ["route", "align", "route_align", "preshuffle", "stage1", "stage2", "forward", "Layer",
           "preshuffle_backward", "backward", "pick_block_m", "align_capacity", "MoEError"]


def _dt(dtype) -> int:
    if dtype in ("bf16", BF16):
        return BF16
    if dtype in ("fp8", FP8):
        return FP8
    if dtype in ("mxfp8", MXFP8):
        return MXFP8
    if dtype in ("mxfp4", MXFP4):
        return MXFP4
    raise ValueError(f"dtype {dtype!r}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def pick_block_m(T: int, k: int, E: int) -> int:
    """M-tile for a batch: 32-row tiles while the mean expert group is at most 24 slots
    (three quarters of a tile, so that few groups spill into a second tile, which would
    stream that expert's weights again), else 128-row tiles. Measured on the Mixtral shape
    (cold cache, FP8): 32 rows are fastest up to T=96 (mean 24), 128 rows from T=128 (mean
    32: 313 us against 376 with 32-row and 320 with 64-row tiles) on."""
    mean = T * k / max(E, 1)
    return 32 if mean <= 24 else 128


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(lib().moe_align_capacity(T, k, E, block_m))


def route(x: torch.Tensor, w_router: torch.Tensor, k: int, bias: torch.Tensor | None = None,
          fp8: bool = False, want_logits: bool = False, mx: bool = False):
    """-> (topk_ids int32 [T,k], topk_w fp32 [T,k], x_q uint8 [T,H] | None,
    x_scale | None, logits fp32 [T,E] | None). x_scale is fp32 [T] with fp8=True, the
    E8M0 block codes uint8 [T, H/32] with mx=True."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    if mx:
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        check(lib().moe_route_mx(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, _ptr(ids),
                                 _ptr(w), _ptr(lg), _ptr(xq), _ptr(xs), _stream()))
        return ids, w, xq, xs, lg
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev) if fp8 else None
    xs = torch.empty((T,), dtype=torch.float32, device=dev) if fp8 else None
    check(lib().moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, _ptr(ids), _ptr(w),
                          _ptr(lg), _ptr(xq), _ptr(xs), _stream()))
    return ids, w, xq, xs, lg


@dataclass
class Grouping:
    """Output of align(): device tensors; only the first `total` rows of sorted_slot are valid."""
    sorted_slot: torch.Tensor
    tile_expert: torch.Tensor
    count: torch.Tensor
    offset: torch.Tensor
    total: torch.Tensor  # int32 [1], on the device
    T: int
    k: int
    E: int
    block_m: int

    @property
    def capacity(self) -> int:
        return self.sorted_slot.numel()


def align(topk_ids: torch.Tensor, E: int, block_m: int) -> Grouping:
    T, k = topk_ids.shape
    cap = align_capacity(T, k, E, block_m)
    if cap < 0:
        check(lib().moe_align(None, T, k, E, block_m, None, None, None, None, None, None))
    dev = topk_ids.device
    ss = torch.empty(cap, dtype=torch.int32, device=dev)
    te = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tot = torch.empty(1, dtype=torch.int32, device=dev)
    check(lib().moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(ss), _ptr(te), _ptr(cnt),
                          _ptr(off), _ptr(tot), _stream()))
    return Grouping(ss, te, cnt, off, tot, T, k, E, block_m)


def route_align(x: torch.Tensor, w_router: torch.Tensor, k: int, block_m: int,
                bias: torch.Tensor | None = None, fp8: bool = False, mx: bool = False,
                want_logits: bool = False):
    """route() then align() of its ids in one call (one launch for a single token):
    -> (topk_ids, topk_w, x_q | None, x_scale | None, logits | None, Grouping)."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev) if fp8 or mx else None
    if mx:
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    else:
        xs = torch.empty((T,), dtype=torch.float32, device=dev) if fp8 else None
    cap = max(align_capacity(T, k, E, block_m), 0)
    g = Grouping(torch.empty(cap, dtype=torch.int32, device=dev),
                 torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev),
                 torch.empty(E + 1, dtype=torch.int32, device=dev),
                 torch.empty(1, dtype=torch.int32, device=dev), T, k, E, block_m)
    check(lib().moe_route_align(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(mx),
                                _ptr(ids), _ptr(w), _ptr(lg), _ptr(xq), _ptr(xs), block_m,
                                _ptr(g.sorted_slot), _ptr(g.tile_expert), _ptr(g.count),
                                _ptr(g.offset), _ptr(g.total), _stream()))
    return ids, w, xq, xs, lg, g


@dataclass
class Weights:
    """Preshuffled expert weights (output of preshuffle())."""
    dtype: int
    E: int
    H: int
    I: int
    w13: torch.Tensor
    w2: torch.Tensor
    s13: torch.Tensor | None
    s2: torch.Tensor | None


def _expert_shape(dt: int, w1) -> tuple[int, int, int]:
    """(E, I, H) from the gate weights (MXFP4 rows hold H/2 bytes)."""
    E, I, Hs = w1.shape
    return E, I, Hs * 2 if dt == MXFP4 else Hs


def preshuffle(dtype, w1, w3, w2, s1=None, s3=None, s2=None) -> Weights:
    dt = _dt(dtype)
    E, I, H = _expert_shape(dt, w1)
    L = lib()
    n13 = L.moe_preshuffle_bytes(dt, E, H, I, 0)
    n2 = L.moe_preshuffle_bytes(dt, E, H, I, 1)
    dev = w1.device
    w13p = torch.empty(n13, dtype=torch.uint8, device=dev)
    w2p = torch.empty(n2, dtype=torch.uint8, device=dev)
    if dt in (MXFP8, MXFP4):  # block codes in the kernels' order (opaque bytes)
        s13p = torch.empty(L.moe_preshuffle_bytes(dt, E, H, I, 2), dtype=torch.uint8, device=dev)
        s2p = torch.empty(L.moe_preshuffle_bytes(dt, E, H, I, 3), dtype=torch.uint8, device=dev)
    else:
        s13p = torch.empty((E, 2, I), dtype=torch.float32, device=dev) if dt == FP8 else None
        s2p = torch.empty((E, H), dtype=torch.float32, device=dev) if dt == FP8 else None
    check(L.moe_preshuffle(dt, E, H, I, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(s1), _ptr(s3),
                           _ptr(s2), _ptr(w13p), _ptr(w2p), _ptr(s13p), _ptr(s2p), _stream()))
    return Weights(dt, E, H, I, w13p, w2p, s13p, s2p)


def stage1(dtype, x_or_xq, x_scale, pw: Weights, grp: Grouping, act=None, act_amax=None):
    """-> (act bf16-bits int16 [capacity, I], act_amax fp32 partial maxima | None)."""
    dt = _dt(dtype)
    T, H = x_or_xq.shape
    I, E, k, bm = pw.I, pw.E, grp.k, grp.block_m
    cap = grp.capacity
    dev = x_or_xq.device
    if act is None:
        act = torch.empty((cap, I), dtype=torch.int16, device=dev)
    if dt == FP8 and act_amax is None:
        n = lib().moe_stage1_amax_floats(dt, T, k, E, H, I, bm)
        act_amax = torch.empty(max(int(n), 0), dtype=torch.float32, device=dev)
    check(lib().moe_stage1(dt, _ptr(x_or_xq), _ptr(x_scale), _ptr(pw.w13), _ptr(pw.s13),
                           _ptr(grp.sorted_slot), _ptr(grp.tile_expert), _ptr(grp.total), T, k,
                           E, H, I, bm, _ptr(act), _ptr(act_amax), _stream()))
    return act, act_amax


def stage2_workspace_bytes(dtype, T, k, E, H, I, block_m) -> int:
    return int(lib().moe_stage2_workspace_bytes(_dt(dtype), T, k, E, H, I, block_m))


def stage2(dtype, act, act_amax, pw: Weights, grp: Grouping, topk_w, out=None, workspace=None):
    """-> out, bf16 bits as int16 [T, H]."""
    dt = _dt(dtype)
    T, k = topk_w.shape
    E, H, I, bm = pw.E, pw.H, pw.I, grp.block_m
    dev = act.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
    nws = stage2_workspace_bytes(dt, T, k, E, H, I, bm)
    if workspace is None:
        workspace = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    check(lib().moe_stage2(dt, _ptr(act), _ptr(act_amax), _ptr(pw.w2), _ptr(pw.s2),
                           _ptr(grp.sorted_slot), _ptr(grp.tile_expert), _ptr(grp.total),
                           _ptr(topk_w), T, k, E, H, I, bm, _ptr(out), _ptr(workspace),
                           workspace.numel(), _stream()))
    return out


def preshuffle_backward(w1, w3, w2):
    """Transposed bf16 weights in the fragment order the backward GEMMs read (load time).
    -> (w2t, w13t) uint8 device tensors."""
    E, I, H = w1.shape
    L = lib()
    w2t = torch.empty(L.moe_backward_preshuffle_bytes(E, H, I, 0), dtype=torch.uint8,
                      device=w1.device)
    w13t = torch.empty(L.moe_backward_preshuffle_bytes(E, H, I, 1), dtype=torch.uint8,
                       device=w1.device)
    check(L.moe_backward_preshuffle(E, H, I, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(w2t), _ptr(w13t),
                                    _stream()))
    return w2t, w13t


def backward(x, w_router, ids, w, grp: Grouping, act, pw: Weights, w2t, w13t, dout,
             want_dbias=True, gu=None):
    """Gradients of sum <dout, out> of the bf16 layer (moe_backward), from the forward's
    tokens x, router weights, routing (ids, w), grouping, stage-1 output act, its saved
    pre-activations gu (Layer(save_preact=True); None: recomputed) and preshuffled
    weights. -> dict(dx, dw1, dw3, dw2, dw_router, dbias), fp32 device tensors."""
    T, H = x.shape
    E, I, k, bm = pw.E, pw.I, grp.k, grp.block_m
    dev = x.device
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = dict(dx=f(T, H), dw1=f(E, I, H), dw3=f(E, I, H), dw2=f(E, H, I), dw_router=f(E, H),
             dbias=f(E) if want_dbias else None)
    L = lib()
    n = int(L.moe_backward_workspace_bytes(T, k, E, H, I, bm))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    check(L.moe_backward(_ptr(x), _ptr(w_router), _ptr(ids), _ptr(w), _ptr(grp.sorted_slot),
                         _ptr(grp.tile_expert), _ptr(grp.offset), _ptr(grp.total), _ptr(act),
                         _ptr(gu), _ptr(pw.w13), _ptr(w2t), _ptr(w13t), _ptr(dout), T, k, E, H,
                         I, bm,
                         _ptr(g["dx"]), _ptr(g["dw1"]), _ptr(g["dw3"]), _ptr(g["dw2"]),
                         _ptr(g["dw_router"]), _ptr(g["dbias"]), _ptr(ws), ws.numel(),
                         _stream()))
    return g


class Layer:
    """The whole routed MoE layer with buffers allocated once for a fixed batch size.

    Weights are preshuffled at construction (load time). __call__ runs route, align,
    stage 1 and stage 2 on the current stream with no host synchronisation. With
    save_preact (bf16 only, for training), stage 1 also keeps the pre-activations g, u in
    self.gu for backward(..., gu=layer.gu)."""

    def __init__(self, dtype, w_router, w1, w3, w2, s1=None, s3=None, s2=None, bias=None,
                 k=2, T=None, block_m=None, save_preact=False):
        self.dt = _dt(dtype)
        if save_preact and self.dt != BF16:
            raise ValueError("save_preact is for the bf16 layer (the backward is bf16)")
        self.save_preact = save_preact
        self.fp8 = self.dt == FP8
        self.mx = self.dt in (MXFP8, MXFP4)
        self.E, self.I, self.H = _expert_shape(self.dt, w1)
        self.k = k
        self.w_router = w_router
        self.bias = bias
        self.pw = preshuffle(self.dt, w1, w3, w2, s1, s3, s2)
        self.T = None
        if T is not None:
            self._alloc(T, block_m)

    def _alloc(self, T, block_m=None):
        E, H, I, k, dev = self.E, self.H, self.I, self.k, self.pw.w13.device
        self.T = T
        self.bm = block_m or pick_block_m(T, k, E)
        cap = align_capacity(T, k, E, self.bm)
        L = lib()
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev) if self.fp8 or self.mx else None
        if self.mx:
            self.xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        else:
            self.xs = torch.empty((T,), dtype=torch.float32, device=dev) if self.fp8 else None
        self.grp = Grouping(torch.empty(cap, dtype=torch.int32, device=dev),
                            torch.empty(cap // self.bm, dtype=torch.int32, device=dev),
                            torch.empty(E, dtype=torch.int32, device=dev),
                            torch.empty(E + 1, dtype=torch.int32, device=dev),
                            torch.empty(1, dtype=torch.int32, device=dev), T, k, E, self.bm)
        self.act = torch.empty((cap, I), dtype=torch.int16, device=dev)
        self.gu = torch.empty((cap, 2 * I), dtype=torch.int16, device=dev) \
            if self.save_preact else None
        n = int(L.moe_stage1_amax_floats(self.dt, T, k, E, H, I, self.bm)) if self.fp8 else 0
        self.amax = torch.empty(max(n, 1), dtype=torch.float32, device=dev) if self.fp8 else None
        nws = stage2_workspace_bytes(self.dt, T, k, E, H, I, self.bm)
        self.ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=torch.int16, device=dev)

    def __call__(self, x: torch.Tensor, events=None) -> torch.Tensor:
        """Run the layer. `events`, if given, is a pair of torch.cuda.Event recorded on the
        current stream right before and after the stage-1 call (a single kernel)."""
        T = x.shape[0]
        if T != self.T:
            self._alloc(T)
        L, st = lib(), _stream()
        E, H, I, k, bm, g = self.E, self.H, self.I, self.k, self.bm, self.grp
        # route + align (one launch for a single-token batch)
        check(L.moe_route_align(_ptr(x), _ptr(self.w_router), _ptr(self.bias), T, H, E, k,
                                int(self.mx), _ptr(self.ids), _ptr(self.w), None, _ptr(self.xq),
                                _ptr(self.xs), bm, _ptr(g.sorted_slot), _ptr(g.tile_expert),
                                _ptr(g.count), _ptr(g.offset), _ptr(g.total), st))
        xin = x if self.dt == BF16 else self.xq
        if events is not None:
            events[0].record()
        if self.save_preact:
            check(L.moe_stage1_save_preact(_ptr(xin), _ptr(self.pw.w13), _ptr(g.sorted_slot),
                                           _ptr(g.tile_expert), _ptr(g.total), T, k, E, H, I,
                                           bm, _ptr(self.act), _ptr(self.gu), st))
        else:
            check(L.moe_stage1(self.dt, _ptr(xin), _ptr(self.xs), _ptr(self.pw.w13),
                               _ptr(self.pw.s13), _ptr(g.sorted_slot), _ptr(g.tile_expert),
                               _ptr(g.total), T, k, E, H, I, bm, _ptr(self.act), _ptr(self.amax),
                               st))
        if events is not None:
            events[1].record()
        check(L.moe_stage2(self.dt, _ptr(self.act), _ptr(self.amax), _ptr(self.pw.w2),
                           _ptr(self.pw.s2), _ptr(g.sorted_slot), _ptr(g.tile_expert),
                           _ptr(g.total), _ptr(self.w), T, k, E, H, I, bm, _ptr(self.out),
                           _ptr(self.ws), self.ws.numel(), st))
        return self.out


    def capture(self, x: torch.Tensor):
        """Capture one layer call on `x` in a HIP graph (torch.cuda.CUDAGraph) and return it.
        `x`'s memory is the graph's input and self.out its output: copy the next batch of
        tokens into x, then graph.replay(). The sequence has no memsets and no host
        synchronisation; every buffer is allocated here, before the capture."""
        T = x.shape[0]
        if T != self.T:
            self._alloc(T)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self(x)  # one call outside the capture first
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self(x)
        return graph


def forward(dtype, x, w_router, w1, w3, w2, s1=None, s3=None, s2=None, bias=None, k=2,
            block_m=None):
    """One-shot layer call (preshuffles the weights each time; use Layer for repeated calls)."""
    return Layer(dtype, w_router, w1, w3, w2, s1, s3, s2, bias, k, x.shape[0], block_m)(x)
