"""Pins of the oracle's grouping of token-slots by expert (counting sort, padding)."""
import numpy as np
import pytest

import oracle


def brute(ids, E, bm):
    T, k = ids.shape
    S = T * k
    slots = sorted(range(S), key=lambda s: (int(ids.flat[s]), s))
    out, tiles = [], []
    for e in range(E):
        grp = [s for s in slots if ids.flat[s] == e]
        pad = -len(grp) % bm
        grp = grp + [S] * pad
        tiles += [e] * (len(grp) // bm)
        out += grp
    return np.array(out, np.int32), np.array(tiles, np.int32)


@pytest.mark.parametrize("T,k,E,bm,seed", [
    (32, 2, 8, 16, 0), (1, 2, 8, 16, 1), (5, 1, 4, 32, 2), (300, 2, 8, 128, 3),
    (64, 8, 8, 16, 4), (257, 3, 64, 64, 5), (0, 2, 8, 16, 6)])
def test_align_matches_bruteforce(T, k, E, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    a = oracle.align(ids, E, bm)
    ss, te = brute(ids, E, bm)
    assert np.array_equal(a["sorted_slot"], ss)
    assert np.array_equal(a["tile_expert"], te)
    assert a["total"] == len(ss) <= oracle.capacity(T, k, E, bm)
    # invariants
    real = a["sorted_slot"][a["sorted_slot"] < T * k]
    assert np.array_equal(np.sort(real), np.arange(T * k))
    assert a["count"].sum() == T * k
    assert np.array_equal(a["count"], np.bincount(ids.ravel(), minlength=E))
    for e in range(E):
        lo, hi = a["offset"][e], a["offset"][e + 1]
        assert lo % bm == 0 and hi % bm == 0
        g = a["sorted_slot"][lo:hi]
        r = g[g < T * k]
        assert np.all(np.diff(r) > 0)
        assert np.all(ids.ravel()[r] == e)
        assert np.all(g[len(r):] == T * k)
        assert hi - lo == -(-a["count"][e] // bm) * bm


def test_align_skewed_all_one_expert():
    T, k, E, bm = 100, 2, 8, 16
    ids = np.zeros((T, k), np.int32)
    ids[:, 1] = 7
    a = oracle.align(ids, E, bm)
    assert a["count"].tolist() == [100, 0, 0, 0, 0, 0, 0, 100]
    assert a["offset"].tolist() == [0, 112, 112, 112, 112, 112, 112, 112, 224]
    assert a["sorted_slot"][:100].tolist() == list(range(0, 200, 2))
    assert a["sorted_slot"][112:212].tolist() == list(range(1, 200, 2))


def test_align_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 9]], np.int32), 8, 16)
