"""Pins for the oracle's context-parallel top-k: one rank's candidates and the merge of all ranks' lists.

Page "DeepSeek V3.2 sparse attention DSA inference flow", pitfalls: with the context split across ranks, each
rank keeps its local top-k candidates and only those are exchanged; the global top-k is chosen from them, which is
exact because a token of the global top-k is also in the local top-k of the rank that holds it.

The pins check that statement itself against the (separately pinned) single-row top-k: splitting a row across
ranks, contiguously or round-robin, and merging the local selections gives exactly the top-k of the whole row
(same indices in the same order, since both use the order value desc, index asc), including rows with ties,
non-finite values and fewer than k valid values.
"""
import numpy as np

import oracle


def _rows(rng, rows, width, kind):
    x = rng.standard_normal((rows, width)).astype(np.float32)
    if kind == "ties":
        x = np.round(x * 2) / 2  # a handful of distinct values
    elif kind == "nonfinite":
        m = rng.random((rows, width))
        x[m < 0.05] = np.inf
        x[(m >= 0.05) & (m < 0.1)] = -np.inf
        x[(m >= 0.1) & (m < 0.15)] = np.nan
    return x.astype(np.float32)


def _split_contiguous(x, ends, R, k):
    rows, W = x.shape
    bounds = np.linspace(0, W, R + 1).astype(np.int32)
    vals, gidx = [], []
    for r in range(R):
        lo, hi = int(bounds[r]), int(bounds[r + 1])
        st = np.full(rows, lo, np.int32)
        en = np.minimum(ends, hi).astype(np.int32)
        idx = oracle.topk_select(x, en, k, starts=st)
        v, g = oracle.topk_values(x, idx, starts=st, index_scale=1, index_offset=lo)
        vals.append(v)
        gidx.append(g)
    return np.stack(vals), np.stack(gidx)


def _split_round_robin(x, ends, R, k):
    rows, W = x.shape
    vals, gidx = [], []
    for r in range(R):
        xr = np.ascontiguousarray(x[:, r::R])
        # rank r holds columns r, r+R, ...: local column c is global c*R + r, valid while c*R + r < end
        en = np.maximum((ends - r + R - 1) // R, 0).astype(np.int32)
        idx = oracle.topk_select(xr, en, k)
        v, g = oracle.topk_values(xr, idx, index_scale=R, index_offset=r)
        vals.append(v)
        gidx.append(g)
    return np.stack(vals), np.stack(gidx)


def test_merge_of_local_topk_is_the_global_topk():
    rng = np.random.default_rng(41)
    for kind in ("plain", "ties", "nonfinite"):
        for R, W, k in ((2, 300, 40), (4, 1000, 64), (8, 4096, 256), (3, 50, 64)):
            x = _rows(rng, 6, W, kind)
            ends = np.array([W, W - 1, W // 2, 7, 0, W], np.int32)
            full = oracle.topk_select(x, ends, k)
            for split in (_split_contiguous, _split_round_robin):
                vals, gidx = split(x, ends, R, k)
                got = oracle.topk_merge(vals, gidx, k)
                assert np.array_equal(got, full), (kind, R, W, k, split.__name__)


def test_values_hand_case():
    logits = np.array([[0.5, -1.0, 2.0, 7.0], [3.0, 4.0, 5.0, 6.0]], np.float32)
    idx = np.array([[2, 0, -1], [1, 2, 9]], np.int32)
    v, g = oracle.topk_values(logits, idx, starts=np.array([1, 0], np.int32), index_scale=4, index_offset=3)
    # row 0 starts at column 1: local 2 -> column 3 (7.0), local 0 -> column 1 (-1.0)
    assert np.array_equal(v, np.array([[7.0, -1.0, -np.inf], [4.0, 5.0, -np.inf]], np.float32))
    assert np.array_equal(g, np.array([[11, 3, -1], [7, 11, -1]], np.int32))


def test_merge_hand_case():
    vals = np.array([[[1.0, 5.0, np.nan]], [[5.0, 9.0, 2.0]]], np.float32)  # 2 lists, 1 row, k_in = 3
    gidx = np.array([[[10, 30, 40]], [[20, -1, 50]]], np.int32)
    # candidates: (1,10) (5,30) (5,20) (2,50); NaN and index -1 ignored
    assert np.array_equal(oracle.topk_merge(vals, gidx, 3), np.array([[20, 30, 50]], np.int32))
    assert np.array_equal(oracle.topk_merge(vals, gidx, 6), np.array([[20, 30, 50, 10, -1, -1]], np.int32))
