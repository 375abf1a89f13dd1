"""Pins for the oracle's top-k selection.

"DeepSeek V3.2 sparse attention DSA inference flow", data flow 2: the indexer writes, per query row, the
2048 best-scoring positions into an int32 table where -1 marks an empty slot; pitfalls section: the
positions are request-relative.  The bf16 variant runs directly on bf16 logits (vLLM PR 56254 summary).
"""
import numpy as np
import torch

import oracle


def values_of(x, idx, starts):
    out = []
    for r in range(idx.shape[0]):
        sel = idx[r][idx[r] >= 0] + (0 if starts is None else starts[r])
        out.append(np.sort(x[r, sel])[::-1])
    return out


def test_value_multiset_matches_torch_topk():
    rng = np.random.default_rng(20)
    x = (rng.standard_normal((6, 3000)) * 10).astype(np.float32)
    x[:, ::7] = np.round(x[:, ::7])  # many exact ties
    ends = np.array([3000, 2500, 2048, 2047, 100, 0], np.int32)
    idx = oracle.topk_select(x, ends, 2048)
    for r in range(6):
        n = min(int(ends[r]), 2048)
        assert np.all(idx[r, :n] >= 0) and np.all(idx[r, n:] == -1)
        if n:
            ref = torch.topk(torch.from_numpy(x[r, :ends[r]]), n).values.numpy()
            assert np.array_equal(np.sort(x[r, idx[r, :n]])[::-1], np.sort(ref)[::-1])
        assert len(set(idx[r, :n].tolist())) == n


def test_order_and_tie_break():
    x = np.array([[1.0, 3.0, 3.0, 2.0, -5.0]], np.float32)
    assert oracle.topk_select(x, np.array([5], np.int32), 3).tolist() == [[1, 2, 3]]
    assert oracle.topk_select(x, np.array([5], np.int32), 7).tolist() == [[1, 2, 3, 0, 4, -1, -1]]


def test_start_offset_gives_relative_positions():
    x = np.array([[9.0, 8.0, 1.0, 2.0, 3.0, 7.0]], np.float32)
    idx = oracle.topk_select(x, np.array([5], np.int32), 2, starts=np.array([2], np.int32))
    assert idx.tolist() == [[2, 1]]  # columns 4 and 3, relative to start 2


def test_non_finite_excluded():
    x = np.array([[np.inf, 1.0, np.nan, -np.inf, 0.5, -2.0]], np.float32)
    idx = oracle.topk_select(x, np.array([6], np.int32), 4)
    assert idx.tolist() == [[1, 4, 5, -1]]


def test_all_equal_and_signed_zero():
    x = np.zeros((1, 10), np.float32)
    x[0, ::2] = -0.0
    idx = oracle.topk_select(x, np.array([10], np.int32), 4)
    assert idx.tolist() == [[0, 1, 2, 3]]  # -0 == +0: ties broken by column


def test_bf16_rows():
    rng = np.random.default_rng(21)
    vals = (rng.standard_normal((3, 500)) * 4).astype(np.float32)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    bits[0, 100:200] = 0xFF80  # -inf: never selected
    ends = np.array([500, 300, 5], np.int32)
    idx = oracle.topk_select(bits, ends, 64, bf16=True)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    for r in range(3):
        n = min(64, int(np.isfinite(f[r, :ends[r]]).sum()))
        ref = torch.topk(torch.from_numpy(np.where(np.isfinite(f[r, :ends[r]]), f[r, :ends[r]], -np.inf)),
                         n).values.numpy()
        assert np.array_equal(np.sort(f[r, idx[r, :n]]), np.sort(ref))
        assert np.all(idx[r, n:] == -1)
    assert not np.any((idx[0] >= 100) & (idx[0] < 200))
