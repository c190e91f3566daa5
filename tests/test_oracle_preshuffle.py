"""Pins of the oracle's preshuffle layout: it is a bijection, and it agrees with
the same layout written as numpy reshapes/transposes (fragments of 16 rows x KE
columns; inside a fragment lane l = 16*q + r holds row r and the q-th quarter
of the KE columns)."""
import numpy as np
import pytest

import oracle


def numpy_layout(w, KE):
    """[R, K] array of elements -> fragment order, via reshape/transpose."""
    R, K = w.shape
    a = w.reshape(R // 16, 16, K // KE, 4, KE // 4)   # rb, r, kb, q, c
    a = a.transpose(0, 2, 3, 1, 4)                    # rb, kb, q, r, c  (lane = 16q + r)
    return np.ascontiguousarray(a).reshape(-1)


@pytest.mark.parametrize("dtype,esize,KE", [("bf16", 2, 32), ("fp8", 1, 128)])
def test_preshuffle_matches_numpy_layout(dtype, esize, KE):
    E, H, I = 3, 256, 384
    rng = np.random.default_rng(2)
    edt = np.uint16 if esize == 2 else np.uint8
    w1 = rng.integers(0, 2 ** (8 * esize), (E, I, H), dtype=np.uint64).astype(edt)
    w3 = rng.integers(0, 2 ** (8 * esize), (E, I, H), dtype=np.uint64).astype(edt)
    w2 = rng.integers(0, 2 ** (8 * esize), (E, H, I), dtype=np.uint64).astype(edt)
    p13, p2 = oracle.preshuffle(dtype, w1, w3, w2)
    ref13, ref2 = [], []
    for e in range(E):
        # composite gate/up rows: blocks of 16 alternating W1, W3
        comp = np.stack([w1[e].reshape(I // 16, 16, H), w3[e].reshape(I // 16, 16, H)], 1)
        ref13.append(numpy_layout(comp.reshape(2 * I, H), KE))
        ref2.append(numpy_layout(w2[e], KE))
    assert np.array_equal(p13.view(edt), np.concatenate(ref13))
    assert np.array_equal(p2.view(edt), np.concatenate(ref2))


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
