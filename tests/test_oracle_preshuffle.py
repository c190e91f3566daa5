"""Pins of the oracle's preshuffle layout: it is a bijection, and it agrees with
the same layout written as numpy reshapes/transposes (fragments of 32 rows x 64
bytes; a fragment is two 1 KB pieces, and in piece pc lane l = 32*h + r holds
row r, bytes 32*h + 16*pc .. +15)."""
import numpy as np
import pytest

import oracle


def numpy_layout(w):
    """[R, K] array of elements -> fragment order, via reshape/transpose of its bytes."""
    R = w.shape[0]
    b = np.ascontiguousarray(w).view(np.uint8).reshape(R, -1)
    Kb = b.shape[1]
    a = b.reshape(R // 32, 32, Kb // 64, 2, 2, 16)    # rb, r, kb, h, pc, byte
    a = a.transpose(0, 2, 4, 3, 1, 5)                 # rb, kb, pc, h, r, byte (lane = 32h + r)
    return np.ascontiguousarray(a).reshape(-1)


@pytest.mark.parametrize("dtype,esize", [("bf16", 2), ("fp8", 1)])
def test_preshuffle_matches_numpy_layout(dtype, esize):
    E, H, I = 3, 256, 384
    rng = np.random.default_rng(2)
    edt = np.uint16 if esize == 2 else np.uint8
    w1 = rng.integers(0, 2 ** (8 * esize), (E, I, H), dtype=np.uint64).astype(edt)
    w3 = rng.integers(0, 2 ** (8 * esize), (E, I, H), dtype=np.uint64).astype(edt)
    w2 = rng.integers(0, 2 ** (8 * esize), (E, H, I), dtype=np.uint64).astype(edt)
    p13, p2 = oracle.preshuffle(dtype, w1, w3, w2)
    ref13, ref2 = [], []
    for e in range(E):
        # composite gate/up rows: blocks of 32 alternating W1, W3
        comp = np.stack([w1[e].reshape(I // 32, 32, H), w3[e].reshape(I // 32, 32, H)], 1)
        ref13.append(numpy_layout(comp.reshape(2 * I, H)))
        ref2.append(numpy_layout(w2[e]))
    assert np.array_equal(p13, np.concatenate(ref13))
    assert np.array_equal(p2, np.concatenate(ref2))


def test_preshuffle_is_a_bijection():
    E, H, I = 2, 256, 256
    n13 = E * I * H
    # distinct labels per element: the output must be a permutation of them
    w1 = np.arange(n13, dtype=np.uint32).reshape(E, I, H)
    w3 = w1 + n13
    w2 = (np.arange(E * H * I, dtype=np.uint32) + 2 * n13).reshape(E, H, I)
    # relabel as bf16-sized elements: use the 16-bit halves of a 32-bit label via two passes
    for half in (0, 1):
        a1 = ((w1 >> (16 * half)) & 0xFFFF).astype(np.uint16)
        a3 = ((w3 >> (16 * half)) & 0xFFFF).astype(np.uint16)
        a2 = ((w2 >> (16 * half)) & 0xFFFF).astype(np.uint16)
        p13, p2 = oracle.preshuffle("bf16", a1, a3, a2)
        if half == 0:
            lo13, lo2 = p13.view(np.uint16).astype(np.uint32), p2.view(np.uint16).astype(np.uint32)
        else:
            lab13 = lo13 | (p13.view(np.uint16).astype(np.uint32) << 16)
            lab2 = lo2 | (p2.view(np.uint16).astype(np.uint32) << 16)
    assert np.array_equal(np.sort(lab13), np.arange(2 * n13, dtype=np.uint32))
    assert np.array_equal(np.sort(lab2), np.arange(2 * n13, 2 * n13 + E * H * I, dtype=np.uint32))
