"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from mixture_experts_routed_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 1 << 20  # a non-null, 256-byte aligned fake address; never dereferenced


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = declared()
    for n in ("moe_route", "moe_align", "moe_preshuffle", "moe_stage1", "moe_stage2"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared()
    assert set(names) == set(_lib.SIGNATURES), "binding signature table out of date"
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = _lib.lib()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    assert L.moe_version().startswith(b"moe-gfx950")


def test_size_queries():
    L = _lib.lib()
    assert L.moe_align_capacity(32, 2, 8, 32) == 320  # ceil((64 + 8*31)/32)*32
    assert L.moe_align_capacity(32, 2, 8, 16) == -1   # block_m below one 32-row fragment
    assert L.moe_align_capacity(8192, 2, 8, 128) == (16384 + 8 * 127 + 127) // 128 * 128
    assert L.moe_align_capacity(8192, 2, 8, 256) == (16384 + 8 * 255 + 255) // 256 * 256
    assert L.moe_align_capacity(1, 2, 8, 48) == -1
    assert L.moe_preshuffle_bytes(1, 8, 4096, 14336, 0) == 2 * 8 * 4096 * 14336
    assert L.moe_preshuffle_bytes(0, 8, 4096, 14336, 1) == 2 * 8 * 4096 * 14336
    assert L.moe_stage1_amax_floats(0, 16, 2, 8, 4096, 14336, 32) == 0
    cap = L.moe_align_capacity(8192, 2, 8, 128)
    # one partial maximum per row and per stage-1 workgroup column block (512 composite rows)
    assert L.moe_stage1_amax_floats(1, 8192, 2, 8, 4096, 14336, 128) == cap * (2 * 14336 // 512)
    # decode tiles (32 rows): 64-row column blocks, 128-row ones where the reduction is
    # split over two waves (one round of workgroups, or every expert live)
    cap4 = L.moe_align_capacity(4, 2, 8, 32)
    assert L.moe_stage1_amax_floats(1, 4, 2, 8, 4096, 14336, 32) == cap4 * (2 * 14336 // 64)
    cap32 = L.moe_align_capacity(16, 2, 8, 32)
    assert L.moe_stage1_amax_floats(1, 16, 2, 8, 4096, 14336, 32) == cap32 * (2 * 14336 // 128)
    cap1 = L.moe_align_capacity(1, 2, 8, 32)
    assert L.moe_stage1_amax_floats(1, 1, 2, 8, 4096, 14336, 32) == cap1 * (2 * 14336 // 128)
    assert L.moe_stage2_workspace_bytes(0, 32, 2, 8, 128, 256, 64) == 64 * 128 * 4
    assert L.moe_stage2_workspace_bytes(1, 3, 2, 8, 128, 256, 32) == -1  # FP8 needs H % 256


def status(fn, *args):
    return getattr(_lib.lib(), fn)(*args)


def test_route_argument_checks():
    S = 0
    args = [FAKE, FAKE, None, 4, 4096, 8, 2, FAKE, FAKE, None, None, None, S]
    assert status("moe_route", *args[:3], -1, *args[4:]) == _lib.ERR_INVALID_ARG
    a = list(args); a[4] = 100
    assert status("moe_route", *a) == _lib.ERR_UNSUPPORTED          # H % 128
    a = list(args); a[6] = 9
    assert status("moe_route", *a) == _lib.ERR_UNSUPPORTED          # k > E
    a = list(args); a[5] = 65
    assert status("moe_route", *a) == _lib.ERR_UNSUPPORTED          # E > 64
    a = list(args); a[0] = None
    assert status("moe_route", *a) == _lib.ERR_INVALID_ARG          # null x
    a = list(args); a[0] = FAKE + 2
    assert status("moe_route", *a) == _lib.ERR_INVALID_ARG          # misaligned x
    a = list(args); a[10] = FAKE
    assert status("moe_route", *a) == _lib.ERR_INVALID_ARG          # x_q without x_scale
    a = list(args); a[3] = 0; a[0] = None
    assert status("moe_route", *a) == _lib.OK                       # T = 0: nothing to do
    assert b"" == _lib.lib().moe_last_error()


def test_align_argument_checks():
    base = [FAKE, 16, 2, 8, 32, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    a = list(base); a[4] = 24
    assert status("moe_align", *a) == _lib.ERR_UNSUPPORTED
    assert b"block_m" in _lib.lib().moe_last_error()
    a = list(base); a[3] = 0
    assert status("moe_align", *a) == _lib.ERR_INVALID_ARG
    a = list(base); a[5] = None
    assert status("moe_align", *a) == _lib.ERR_INVALID_ARG
    a = list(base); a[1] = 0
    assert status("moe_align", *a) == _lib.OK


def test_route_align_argument_checks():
    # x, w_router, bias, T, H, E, k, mx, ids, w, logits, x_q, x_scale, block_m,
    # sorted_slot, tile_expert, count, offset, total, stream
    base = [FAKE, FAKE, None, 4, 4096, 8, 2, 0, FAKE, FAKE, None, FAKE, FAKE, 32,
            FAKE, FAKE, FAKE, FAKE, FAKE, None]
    a = list(base); a[7] = 2
    assert status("moe_route_align", *a) == _lib.ERR_INVALID_ARG      # mx is 0 or 1
    a = list(base); a[13] = 48
    assert status("moe_route_align", *a) == _lib.ERR_UNSUPPORTED      # block_m
    a = list(base); a[4] = 100
    assert status("moe_route_align", *a) == _lib.ERR_UNSUPPORTED      # H % 128
    a = list(base); a[6] = 9
    assert status("moe_route_align", *a) == _lib.ERR_UNSUPPORTED      # k > E
    a = list(base); a[7] = 1; a[11] = None; a[12] = None
    assert status("moe_route_align", *a) == _lib.ERR_INVALID_ARG      # MX needs x_q, scales
    a = list(base); a[12] = None
    assert status("moe_route_align", *a) == _lib.ERR_INVALID_ARG      # x_q without x_scale
    a = list(base); a[16] = None
    assert status("moe_route_align", *a) == _lib.ERR_INVALID_ARG      # null grouping output
    a = list(base); a[1] = FAKE + 4
    assert status("moe_route_align", *a) == _lib.ERR_INVALID_ARG      # misaligned w_router
    a = list(base); a[3] = 0; a[0] = None; a[14] = None
    assert status("moe_route_align", *a) == _lib.OK                  # T = 0: nothing to do


def test_preshuffle_argument_checks():
    base = [1, 8, 4096, 14336, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    a = list(base); a[0] = 7
    assert status("moe_preshuffle", *a) == _lib.ERR_INVALID_ARG
    a = list(base); a[3] = 14336 + 128
    assert status("moe_preshuffle", *a) == _lib.ERR_UNSUPPORTED     # FP8 needs I % 256
    a = list(base); a[7] = None
    assert status("moe_preshuffle", *a) == _lib.ERR_INVALID_ARG     # FP8 scale missing
    a = list(base); a[10] = FAKE + 4
    assert status("moe_preshuffle", *a) == _lib.ERR_INVALID_ARG     # misaligned output


def stage2_args(ws_bytes, T=16):
    return [1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, 2, 8, 4096, 14336, 32, FAKE,
            FAKE, ws_bytes, None]


def test_stage_argument_checks():
    s1 = [1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 8, 4096, 14336, 32, FAKE, FAKE, None]
    for bad_bm in (16, 48, 512):
        a = list(s1); a[13] = bad_bm
        assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED     # block_m
    a = list(s1); a[15] = None
    assert status("moe_stage1", *a) == _lib.ERR_INVALID_ARG         # FP8 without act_amax
    a = list(s1); a[9] = 9
    assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED         # k > 8
    # the training forward's stage 1 (bf16): gu is required and 16-byte aligned
    sp = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 8, 4096, 14336, 32, FAKE, FAKE, None]
    a = list(sp); a[12] = None
    assert status("moe_stage1_save_preact", *a) == _lib.ERR_INVALID_ARG
    a = list(sp); a[12] = FAKE + 8
    assert status("moe_stage1_save_preact", *a) == _lib.ERR_INVALID_ARG
    a = list(sp); a[10] = 48
    assert status("moe_stage1_save_preact", *a) == _lib.ERR_UNSUPPORTED   # block_m
    need = _lib.lib().moe_stage2_workspace_bytes(1, 16, 2, 8, 4096, 14336, 32)
    assert need >= 16 * 2 * 4096 * 4
    assert status("moe_stage2", *stage2_args(need - 1)) == _lib.ERR_WORKSPACE
    a = stage2_args(need); a[16] = FAKE + 16
    assert status("moe_stage2", *a) == _lib.ERR_INVALID_ARG         # workspace alignment
    assert status("moe_stage2", *stage2_args(0, T=0)) == _lib.OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_mxfp8_size_queries_and_checks():
    L = _lib.lib()
    E, H, I = 8, 4096, 14336
    assert L.moe_preshuffle_bytes(2, E, H, I, 0) == 2 * E * I * H            # one byte per value
    assert L.moe_preshuffle_bytes(2, E, H, I, 2) == 2 * E * I * (H // 32)    # one code per 32
    assert L.moe_preshuffle_bytes(2, E, H, I, 3) == E * H * (I // 32)
    assert L.moe_preshuffle_bytes(1, E, H, I, 2) == 2 * E * I * 4            # fp32 per row
    assert L.moe_preshuffle_bytes(0, E, H, I, 3) == 0
    assert L.moe_stage1_amax_floats(2, 8192, 2, E, H, I, 128) == 0          # no row maxima
    cap = L.moe_align_capacity(16, 2, E, 32)
    need = L.moe_stage2_workspace_bytes(2, 16, 2, E, H, I, 32)
    up = lambda b: (b + 255) // 256 * 256
    assert need >= up(16 * 2 * H * 4) + up(cap * I) + up(cap * I // 32)
    # MXFP8 limits: H <= 8192 (stage 1 token-code tile), I <= 16384
    s1 = [2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 8, 4096, 14336, 32, FAKE, None, None]
    a = list(s1); a[11] = 8192 + 256
    assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED
    a = list(s1); a[12] = 16384 + 256
    assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED
    a = list(s1); a[2] = None
    assert status("moe_stage1", *a) == _lib.ERR_INVALID_ARG          # block codes of x missing
    a = list(s1); a[2] = FAKE + 4
    assert status("moe_stage1", *a) == _lib.ERR_INVALID_ARG          # x codes 8-byte aligned
    r = [FAKE, FAKE, None, 4, 4096, 8, 2, FAKE, FAKE, None, FAKE, None, None]
    assert status("moe_route_mx", *r) == _lib.ERR_INVALID_ARG         # codes output missing
    a = list(r); a[4] = 4096 + 64
    assert status("moe_route_mx", *a) == _lib.ERR_UNSUPPORTED         # H % 128
    a = list(r); a[3] = 0; a[10] = None
    assert status("moe_route_mx", *a) == _lib.OK


def test_mxfp4_size_queries_and_checks():
    L = _lib.lib()
    E, H, I = 8, 4096, 14336
    assert L.moe_preshuffle_bytes(3, E, H, I, 0) == E * I * H                # two values per byte
    assert L.moe_preshuffle_bytes(3, E, H, I, 1) == E * H * I // 2
    assert L.moe_preshuffle_bytes(3, E, H, I, 2) == 2 * E * I * (H // 32)    # one code per 32
    assert L.moe_preshuffle_bytes(3, E, H, I, 3) == E * H * (I // 32)
    assert L.moe_preshuffle_bytes(4, E, H, I, 0) == -1                        # no such dtype
    assert L.moe_stage1_amax_floats(3, 8192, 2, E, H, I, 128) == 0
    cap = L.moe_align_capacity(16, 2, E, 32)
    need = L.moe_stage2_workspace_bytes(3, 16, 2, E, H, I, 32)
    up = lambda b: (b + 255) // 256 * 256
    assert need >= up(16 * 2 * H * 4) + up(cap * I) + up(cap * I // 32)
    s1 = [3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 8, 4096, 14336, 32, FAKE, None, None]
    a = list(s1); a[11] = 8192 + 256
    assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED          # H <= 8192
    a = list(s1); a[12] = 16384 + 256
    assert status("moe_stage1", *a) == _lib.ERR_UNSUPPORTED          # I <= 16384
    a = list(s1); a[4] = None
    assert status("moe_stage1", *a) == _lib.ERR_INVALID_ARG          # weight codes missing
    p = [3, 8, 4096, 14336, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    assert status("moe_preshuffle", *p) == _lib.ERR_INVALID_ARG      # scales required
    a = [4] + s1[1:]
    assert status("moe_stage1", *a) == _lib.ERR_INVALID_ARG          # unknown dtype


def test_pick_block_m_rule():
    # 32-row tiles while the mean expert group is at most 24 slots, else 128-row tiles
    import mixture_experts_routed_top_amd as moe
    assert [moe.pick_block_m(T, 2, 8) for T in (1, 16, 64, 96)] == [32] * 4
    assert [moe.pick_block_m(T, 2, 8) for T in (97, 128, 256, 8192)] == [128] * 4
    assert moe.pick_block_m(12, 1, 1) == 32 and moe.pick_block_m(25, 1, 1) == 128
    for T in (1, 96, 97, 8192):  # every choice has a capacity the align call accepts
        assert moe.align_capacity(T, 2, 8, moe.pick_block_m(T, 2, 8)) > 0
