"""Shared helpers for the GPU parity tests: device transfer, the tolerance rules and the top-k comparison.

Tolerances (the indexer's stated bar): fp32 logits |gpu - ref| <= 1e-3 (1 + |ref|); bf16 sparse logits add
half a bf16 ulp, 2^-8 |ref|, for the one rounding the path performs.  A top-k selection is accepted when it
has the oracle's size and every swap is within one tolerance: for a selected g and a non-selected valid x,
ref[x] - ref[g] <= 1e-3 (1 + max(|ref[x]|, |ref[g]|)).  On bf16 rows each side's half ulp is added, since two
logits that differ by up to one bf16 ulp can round to the same value and tie.
"""
import concurrent.futures
import os

import numpy as np
import torch

import oracle

ROW = 132


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def tol_f32(ref):
    return 1e-3 * (1.0 + np.abs(ref))


def tol_bf16(ref):
    return 1e-3 * (1.0 + np.abs(ref)) + 2.0 ** -8 * np.abs(ref)


def bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_close(gpu, ref, tol_fn=tol_f32, what="logits"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = ~(err <= tol_fn(ref))
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {i.tolist()} "
                             f"gpu={gpu[bad][:5]} ref={ref[bad][:5]}")


def swap_tolerance(x, g, rule="f32"):
    """Largest ref[x] - ref[g] allowed when g is selected and x is not (element-wise).  rule: "f32" (one logit
    tolerance), "bf16" (plus each side's half ulp) or "exact" (identical inputs: no swap across a difference)."""
    x, g = np.abs(np.asarray(x, np.float64)), np.abs(np.asarray(g, np.float64))
    if rule == "exact":
        return 0.0 * (x + g)
    t = 1e-3 * (1.0 + np.maximum(x, g))
    if rule == "bf16":
        return t + 2.0 ** -8 * (x + g)
    assert rule == "f32", rule
    return t


def check_selection(gpu_idx, ref_idx, ref_vals, rule="f32", start=0, end=None):
    """One row.  gpu_idx/ref_idx: int32 [k] positions relative to `start` (-1 = empty); ref_vals: the oracle's
    values of the row (absolute columns).  Same size, no duplicates, valid positions, and every swap within
    swap_tolerance(rule)."""
    end = ref_vals.shape[0] if end is None else end
    g = gpu_idx[gpu_idx >= 0]
    o = ref_idx[ref_idx >= 0]
    assert g.size == o.size, (g.size, o.size)
    assert np.all(gpu_idx[g.size:] == -1), "valid entries must come first, then -1"
    assert np.unique(g).size == g.size, "duplicate selection"
    cols = g + start
    assert np.all((cols >= start) & (cols < end)), "selection outside the row range"
    row = ref_vals[start:end].astype(np.float64)
    finite = np.isfinite(row)
    sel = np.zeros(row.shape, dtype=bool)
    sel[g] = True
    assert np.all(finite[g]), "selected a non-finite value"
    if g.size == 0:
        assert finite.sum() == 0
        return
    rest = finite & ~sel
    if not rest.any():
        return
    rv, sv = row[rest], row[g]
    lo = sv.min()
    hi = rv.max()
    if hi <= lo:
        return
    # only pairs ordered the wrong way need a check: non-selected above the smallest selected value, and
    # selected below the largest non-selected value
    xs = rv[rv > lo]
    gs = sv[sv < hi]
    diff = xs[:, None] - gs[None, :]
    ok = diff <= swap_tolerance(xs[:, None], gs[None, :], rule)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"selection misses a larger value: non-selected {xs[i]} vs selected {gs[j]} "
                             f"(difference {diff[i, j]}, allowed {swap_tolerance(xs[i], gs[j], rule)})")


def gathered_rows_oracle(k_bf16):
    """Oracle quantization of contiguous tokens into gathered cache rows [S,132]."""
    S = k_bf16.shape[0]
    rows = np.zeros((S, ROW), np.uint8)
    oracle.k_quant_and_cache(k_bf16, np.arange(S), rows.reshape(-1), max(S, 1), max(S, 1) * ROW)
    return rows


def paged_pool_oracle(k_bf16, slot_mapping, num_blocks, block_size, block_stride):
    pool = np.zeros(num_blocks * block_stride, np.uint8)
    oracle.k_quant_and_cache(k_bf16, slot_mapping, pool, block_size, block_stride)
    return pool


def parallel(fn, items, workers=None):
    """fn(item) for every item on host threads, re-raising the first failure.  The oracle's C calls release the
    interpreter lock, so its single-threaded instances run side by side (at most 16, the host share of one GPU)."""
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(fn, it) for it in items]:
            f.result()
