"""Pins of the oracle's token -> expert align (histogram, prefix scan, padded-block permutation)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_handworked():
    g = json.load(open(os.path.join(GOLD, "align_handworked.json")))
    s, b, n = oracle.align_block(np.array(g["topk_ids"]), g["E"], g["block_m"])
    np.testing.assert_array_equal(s, g["sorted_ids"])
    np.testing.assert_array_equal(b, g["block_expert"])
    assert n == g["num_padded"]


@pytest.mark.parametrize("T,k,E,bm", [(1, 1, 1, 16), (16, 2, 8, 16), (37, 6, 64, 16), (64, 2, 8, 32),
                                      (5, 8, 128, 64), (100, 3, 4, 1), (33, 2, 8, 128)])
def test_bruteforce_and_invariants(T, k, E, bm):
    rng = np.random.default_rng(T * 1000 + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if E > 4:
        ids[: T // 2, 0] = 0          # skew one expert
    s, b, n = oracle.align_block(ids, E, bm)
    s2, b2, n2 = oracle.align_block_bruteforce(ids, E, bm)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(b, b2)
    assert n == n2
    tk = T * k
    assert s.size == oracle.align_capacity(T, k, E, bm) and s.size % bm == 0
    # each flat index exactly once
    real = s[s < tk]
    np.testing.assert_array_equal(np.sort(real), np.arange(tk))
    counts = np.bincount(ids.ravel(), minlength=E)
    assert n == int((-(-counts // bm) * bm).sum())
    assert int((s[:n] == tk).sum()) == n - tk
    assert np.all(s[n:] == tk)
    # blocks: expert non-decreasing, and every row of a block belongs to its expert
    nb = n // bm
    assert np.all(np.diff(b[:nb]) > -1) and np.all(b[nb:] == -1)
    flat = ids.ravel()
    for blk in range(nb):
        rows = s[blk * bm:(blk + 1) * bm]
        rows = rows[rows < tk]
        assert rows.size > 0
        assert np.all(flat[rows] == b[blk])
        assert np.all(np.diff(rows) > 0)   # stable: ascending inside the block


def test_out_of_range_ids_dropped():
    ids = np.array([[0, 9], [-1, 1], [1, 0]], np.int32)
    s, b, n = oracle.align_block(ids, 2, 2)
    assert n == 4
    np.testing.assert_array_equal(s[:4], [0, 5, 3, 4])
    assert set(s[4:].tolist()) <= {6}


def test_capacity_is_tight():
    # the worst case fills the capacity exactly: every non-empty expert has one row over a block
    E, bm = 4, 8
    ids = np.repeat(np.arange(E), bm + 1)
    s, b, n = oracle.align_block(ids.reshape(-1, 1), E, bm)
    assert n == E * 2 * bm
    assert n == s.size
