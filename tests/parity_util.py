"""Shared helpers for the GPU parity tests: device transfer, the tolerance rules and the top-k comparison.

Tolerances (the indexer's stated bar): fp32 logits |gpu - ref| <= 1e-3 (1 + |ref|); bf16 sparse logits add
half a bf16 ulp, 2^-8 |ref|, for the one rounding the path performs; a top-k selection is accepted when it
has the oracle's size and every selected/non-selected pair is ordered correctly up to those tolerances.
"""
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


def check_selection(gpu_idx, ref_idx, ref_vals, tol_fn=tol_f32, start=0, end=None):
    """One row.  gpu_idx/ref_idx: int32 [k] positions relative to `start` (-1 = empty); ref_vals: the oracle's
    values of the row (absolute columns).  Same size, no duplicates, valid positions, and
    max over non-selected valid x of (ref[x] - tol) <= min over selected g of (ref[g] + tol)."""
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
    if rest.any():
        hi_rest = np.max(row[rest] - tol_fn(row[rest]))
        lo_sel = np.min(row[g] + tol_fn(row[g]))
        assert hi_rest <= lo_sel, f"selection misses a larger value: {hi_rest} > {lo_sel}"


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
