"""Pins of the oracle's large-k top-k (the sparse attention indexer's
selection), no GPU: numpy's lexsort under the same total order, hand-built
boundary cases, and the padding rule for short rows."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle as O


def np_topk(scores, k, lengths=None):
    """numpy reference: order by (NaN last, value descending with -0 == +0,
    index ascending) over the first lengths[q] entries; -1 padding."""
    Q, N = scores.shape
    idx = np.full((Q, k), -1, dtype=np.int32)
    for q in range(Q):
        n = N if lengths is None else min(max(int(lengths[q]), 0), N)   # clamped to [0, N]
        row = scores[q, :n].astype(np.float64) + 0.0          # -0 -> +0
        nan = np.isnan(row)
        val = np.where(nan, 0.0, row)
        order = np.lexsort((np.arange(n), -val, nan))
        m = min(k, n)
        idx[q, :m] = order[:m]
    return idx


def _quantised_rows(rng, Q, N, levels):
    s = rng.integers(0, levels, size=(Q, N)).astype(np.float32) * np.float32(0.25) - 1.0
    return s


@pytest.mark.parametrize("Q,N,k,levels", [(6, 1000, 100, 7), (4, 4096, 2048, 50),
                                          (3, 131072, 2048, 1000), (5, 300, 300, 3)])
def test_topk_large_equals_lexsort(Q, N, k, levels):
    rng = np.random.default_rng(N + k)
    s = _quantised_rows(rng, Q, N, levels)          # heavy ties
    s[0, rng.choice(N, N // 10, replace=False)] = np.nan
    s[1, : min(N, 5)] = np.inf
    s[1, 5:10] = -np.inf
    s[2, ::7] = -0.0
    s[2, 1::7] = 0.0
    idx, vals = O.topk_large(s, k)
    assert np.array_equal(idx, np_topk(s, k))
    got = np.take_along_axis(s, np.maximum(idx, 0), axis=1)
    assert np.array_equal(vals.view(np.uint32)[idx >= 0], got.view(np.uint32)[idx >= 0])


def test_topk_large_row_lengths_and_padding():
    rng = np.random.default_rng(2)
    Q, N, k = 8, 3000, 2048
    s = rng.standard_normal((Q, N)).astype(np.float32)
    lengths = np.array([0, 1, -1, 2047, 2048, 2049, 3000, -100], dtype=np.int32)
    idx, vals = O.topk_large(s, k, lengths)
    assert np.array_equal(idx, np_topk(s, k, lengths))
    for q, n in enumerate(np.maximum(lengths, 0)):
        assert np.all(idx[q, min(k, n):] == -1)
        assert np.all(np.isnan(vals[q, min(k, n):]))
        assert np.all(idx[q, :min(k, n)] < n)


def test_topk_large_hand_cases():
    # all equal: the lowest indices in order
    idx, _ = O.topk_large(np.zeros((1, 10), np.float32), 4)
    assert idx.tolist() == [[0, 1, 2, 3]]
    # a tie straddling the boundary: the lower index wins, in both index orders
    idx, _ = O.topk_large(np.array([[1.0, 2.0, 1.0, 3.0]], np.float32), 3)
    assert idx.tolist() == [[3, 1, 0]]
    idx, _ = O.topk_large(np.array([[3.0, 1.0, 2.0, 1.0]], np.float32), 3)
    assert idx.tolist() == [[0, 2, 1]]
    # one ulp apart: the larger wins
    a = np.float32(1.5)
    b = np.nextafter(a, np.float32(-np.inf))
    idx, _ = O.topk_large(np.array([[b, a]], np.float32), 1)
    assert idx.tolist() == [[1]]
    # -0 == +0 (ties by index), NaN after -inf, NaNs by index
    s = np.array([[np.nan, -0.0, -np.inf, 0.0, np.nan]], np.float32)
    idx, _ = O.topk_large(s, 5)
    assert idx.tolist() == [[1, 3, 2, 0, 4]]
    # k = N and k = 1
    s = np.array([[0.5, -2.0, 7.0]], np.float32)
    assert O.topk_large(s, 3)[0].tolist() == [[2, 0, 1]]
    assert O.topk_large(s, 1)[0].tolist() == [[2]]
