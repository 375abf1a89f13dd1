"""The five workloads end to end on the GPU, at their full sizes, in the launch configuration the bench times.

The GPU runs every step for every row; the oracle recomputes every row (workloads 1-5) from the same generator
inputs (its own quantized K, never bytes produced by the GPU), its single-threaded instances side by side on
the host's threads.  Workloads:
  1 tiny dense indexer (T=8 at positions 3064..3071, S=3072),
  2 prefill chunk (T=2048 at 6144..8191, S=8192),
  3 paged decode (64 requests, lengths U{4096..65536}, 64-token pages, random block tables),
  4 long-context decode (16 requests x next_n 2, lengths U{98304..131072}),
  5 hierarchical sparse (32 decode requests + a 1024-row prefill chunk, lengths U{32768..131072},
    64 candidate blocks of 128 tokens per row with duplicates and out-of-range ids).
Decode workloads run the fused decode call (logits and top-k in one call), as the bench does.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_amd as dsi
import synth
from parity_util import (ROW, assert_close, bf16_value, check_selection, dev, gathered_rows_oracle, host, parallel,
                         tol_bf16)

pytestmark = pytest.mark.gpu
K = 2048


def _gpu_gathered_rows(k_bf16):
    S = k_bf16.shape[0]
    rows = torch.zeros((S, ROW), dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache(dev(k_bf16), dev(np.arange(S, dtype=np.int64)), rows.view(-1), S, S * ROW, 1)
    return rows


def _prefill_workload(n):
    c = synth.workload(n)
    T, S = c["T"], c["S"]
    rows_ref = gathered_rows_oracle(c["k"])
    rows_gpu = _gpu_gathered_rows(c["k"])
    assert np.array_equal(host(rows_gpu), rows_ref), "k quantization is not bit-exact"
    ks, ke = c["ks"], c["ke"]
    logits = dsi.mqa_logits_prefill(dev(c["q"]), dev(c["w"]), rows_gpu, dev(ks), dev(ke))
    idx = host(dsi.topk_select(logits, dev(ke), k=K, row_starts=dev(ks)))
    got = host(logits)

    def check(t0):
        for t in range(t0, min(t0 + 32, T)):
            ref = oracle.mqa_logits_gathered(c["q"][t:t + 1], c["w"][t:t + 1], rows_ref, ks[t:t + 1], ke[t:t + 1])[0]
            valid = np.isfinite(ref)
            assert_close(got[t][valid], ref[valid], what=f"row {t} logits")
            ref_idx = oracle.topk_select(ref[None, :], ke[t:t + 1], K, starts=ks[t:t + 1])[0]
            check_selection(idx[t], ref_idx, ref, start=ks[t], end=ke[t])

    parallel(check, range(0, T, 32))
    return c, got, idx


def test_workload1_tiny_dense():
    c, got, idx = _prefill_workload(1)
    # identical-input top-k: GPU selection over the oracle's own logits has the oracle's exact value multiset
    rows_ref = gathered_rows_oracle(c["k"])
    ref = oracle.mqa_logits_gathered(c["q"], c["w"], rows_ref, c["ks"], c["ke"])
    same = host(dsi.topk_select(dev(ref), dev(c["ke"]), k=K))
    ref_idx = oracle.topk_select(ref, c["ke"], K)
    for t in range(8):
        assert np.array_equal(np.sort(ref[t, same[t][same[t] >= 0]]), np.sort(ref[t, ref_idx[t][ref_idx[t] >= 0]]))


def test_workload2_prefill_chunk():
    _prefill_workload(2)


def _decode_workload(n, mxfp4=False):
    c = synth.workload(n)
    bs, nb = c["block_size"], c["num_blocks"]
    row = 68 if mxfp4 else ROW
    stride = bs * row if mxfp4 else c["block_stride"]
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    quant_ref = oracle.k_quant_and_cache_mxfp4 if mxfp4 else oracle.k_quant_and_cache
    logits_ref = oracle.mqa_logits_paged_mxfp4 if mxfp4 else oracle.mqa_logits_paged
    nn, B = c["next_n"], c["B"]
    lens = c["context_lens"]
    maxc = int(lens.max())
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    quant(dev(c["k"]), dev(c["slot_mapping"]), pool, bs, stride, nb)
    bt = dev(c["block_table"])
    logits, idx_t = dsi.paged_mqa_topk_decode(dev(c["q"]), dev(c["w"]), dev(lens), pool, bs, bt, maxc, next_n=nn,
                                              k=K, block_stride_bytes=stride, num_blocks=nb, mxfp4=mxfp4)
    ends = np.repeat(lens, nn) - nn + np.tile(np.arange(nn), B) + 1
    row_to_req = np.repeat(np.arange(B, dtype=np.int32), nn)
    slots = host(dsi.req_index_to_global_slot(idx_t, bt, bs, bs, row_to_req=dev(row_to_req)))
    idx = host(idx_t)
    got = host(logits)
    pool_gpu = host(pool)
    starts = np.concatenate([[0], np.cumsum(lens)])

    def check(b):
        L = int(lens[b])
        nblk = (L + bs - 1) // bs
        # the oracle quantizes this request's tokens into a pool of its own (pages in order) ...
        pool_ref = np.zeros(nblk * bs * row, np.uint8)
        quant_ref(c["k"][starts[b]:starts[b + 1]], np.arange(L, dtype=np.int64), pool_ref, bs, bs * row)
        # ... whose rows equal the GPU's rows of the same tokens, found through the request's block table
        toks = (c["block_table"][b, np.arange(L) // bs].astype(np.int64) * stride + (np.arange(L) % bs) * row)
        assert np.array_equal(pool_gpu[toks[:, None] + np.arange(row)[None, :]], pool_ref.reshape(-1, row)[:L]), \
            f"request {b}: k rows differ"
        rr = slice(b * nn, (b + 1) * nn)
        ref = logits_ref(c["q"][rr], c["w"][rr], nn, lens[b:b + 1], pool_ref, bs, bs * row,
                         np.arange(nblk, dtype=np.int32)[None, :], maxc)
        for i in range(nn):
            r = b * nn + i
            valid = np.isfinite(ref[i])
            assert_close(got[r][valid], ref[i][valid], what=f"row {r} logits")
            assert valid.sum() == ends[r]
            ref_idx = oracle.topk_select(ref[i:i + 1], ends[r:r + 1], K)[0]
            check_selection(idx[r], ref_idx, ref[i], end=int(ends[r]))
            if int(ends[r]) < K:
                assert np.all(idx[r][int(ends[r]):] == -1)
            # slot conversion of the selected positions through the request's block table
            p = idx[r]
            exp = np.where(p >= 0, c["block_table"][b, np.maximum(p, 0) // bs] * bs + np.maximum(p, 0) % bs, -1)
            assert np.array_equal(slots[r], exp)

    parallel(check, range(B))


def test_workload3_paged_decode():
    _decode_workload(3)


def test_workload4_long_context_decode():
    _decode_workload(4)


def test_workload3_paged_decode_mxfp4():
    """Workload 3 on the MXFP4 cache: quantize into 68-byte rows, score, select, convert to slots."""
    _decode_workload(3, mxfp4=True)


def test_workload4_long_context_decode_mxfp4():
    _decode_workload(4, mxfp4=True)


def _sparse_workload(mxfp4):
    """Workload 5 (FP8 or MXFP4 cache): expansion, sparse logits (decode requests from the paged pool of 128-token
    pages, the prefill request gathered), bf16 top-k, remap, slots; every row against the oracle."""
    c = synth.workload(5)
    sbk, cbs, nd, rows = c["sbk"], c["cbs"], c["n_decode"], c["rows"]
    bs, nb = c["block_size"], c["num_blocks"]
    row = 68 if mxfp4 else ROW
    stride = bs * row
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    quant_ref = oracle.k_quant_and_cache_mxfp4 if mxfp4 else oracle.k_quant_and_cache
    logits_fn = dsi.sparse_mqa_logits_mxfp4 if mxfp4 else dsi.sparse_mqa_logits
    logits_ref = oracle.sparse_mqa_logits_mxfp4 if mxfp4 else oracle.sparse_mqa_logits
    ks, ke, cand = c["ks"], c["ke"], c["cand"]
    # expansion for every row: bit-exact
    si_ref, end_ref = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    si_t, end_t = dsi.expand_candidates(dev(cand), dev(ks), dev(ke), cbs, sbk)
    assert np.array_equal(host(si_t), si_ref) and np.array_equal(host(end_t), end_ref)
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    quant(dev(c["k_dec"]), dev(c["dec_slot_mapping"]), pool, bs, stride, nb)
    Lp = c["Lp"]
    pre = torch.zeros(Lp * row, dtype=torch.uint8, device="cuda")
    quant(dev(c["k_pre"]), dev(np.arange(Lp, dtype=np.int64)), pre, Lp, Lp * row, 1)
    pre_ref = np.zeros(Lp * row, np.uint8)
    quant_ref(c["k_pre"], np.arange(Lp, dtype=np.int64), pre_ref, Lp, Lp * row)
    assert np.array_equal(host(pre), pre_ref), "prefill k rows differ"
    width = si_ref.shape[1] * sbk
    out = torch.empty((rows, width), dtype=torch.int16, device="cuda")
    q, w, ks_t, ke_t, bt = dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(c["block_table"])
    r2r = dev(c["row_to_req"])
    logits_fn(q[:nd], w[:nd], ks_t[:nd], ke_t[:nd], si_t[:nd], end_t[:nd], sbk, pool, block_table=bt, row_to_req=r2r,
              block_size=bs, block_stride_bytes=stride, num_k=nb, out=out[:nd])
    logits_fn(q[nd:], w[nd:], ks_t[nd:], ke_t[nd:], si_t[nd:], end_t[nd:], sbk, pre, num_k=Lp, out=out[nd:])
    col_t = dsi.topk_select(out, end_t, k=K)
    pos_t = dsi.topk_remap(col_t, si_t, ks_t, sbk)
    slot_t = dsi.req_index_to_global_slot(pos_t[:nd], bt, bs, bs, row_to_req=r2r)
    got, col, pos, slot = host(out), host(col_t), host(pos_t), host(slot_t)
    pool_gpu = host(pool)
    starts = np.concatenate([[0], np.cumsum(c["dec_lens"])])

    def check(r0):
        for r in range(r0, min(r0 + 16, rows)):
            if r < nd:
                L = int(c["dec_lens"][r])
                nblk = (L + bs - 1) // bs
                pool_ref = np.zeros(nblk * stride, np.uint8)
                quant_ref(c["k_dec"][starts[r]:starts[r + 1]], np.arange(L, dtype=np.int64), pool_ref, bs, stride)
                toks = c["block_table"][r, np.arange(L) // bs].astype(np.int64) * stride + (np.arange(L) % bs) * row
                assert np.array_equal(pool_gpu[toks[:, None] + np.arange(row)[None, :]],
                                      pool_ref.reshape(-1, row)[:L]), f"request {r}: k rows differ"
                kw = dict(k_src=pool_ref, block_table=np.arange(nblk, dtype=np.int32)[None, :],
                          row_to_req=np.zeros(1, np.int32), block_size=bs, block_stride=stride)
            else:
                kw = dict(k_src=pre_ref)
            sl = slice(r, r + 1)
            ref_f32 = logits_ref(c["q"][sl], c["w"][sl], ks[sl], ke[sl], si_ref[sl], end_ref[sl], sbk, out_f32=True,
                                 **kw)[0]
            ref_bits = logits_ref(c["q"][sl], c["w"][sl], ks[sl], ke[sl], si_ref[sl], end_ref[sl], sbk, **kw)[0]
            valid = np.isfinite(ref_f32)
            assert np.all(got[r][~valid] == 0xFF80)
            assert_close(bf16_value(got[r][valid]), ref_f32[valid], tol_fn=tol_bf16, what=f"row {r} sparse logits")
            ref_col = oracle.topk_select(ref_bits[None, :], end_ref[sl], K, bf16=True)[0]
            check_selection(col[r], ref_col, ref_f32, rule="bf16", end=int(end_ref[r]))
            # remap (every row) and slots (decode rows) bit-exact against the oracle on the GPU's columns
            assert np.array_equal(pos[r], oracle.topk_remap(col[sl], si_ref[sl], ks[sl], sbk)[0])
            if r < nd:
                exp = oracle.req_index_to_global_slot(pos[sl], c["block_table"], bs, bs,
                                                      row_to_req=c["row_to_req"][sl])[0]
                assert np.array_equal(slot[r], exp)

    parallel(check, range(0, rows, 16))


@pytest.mark.parametrize("mxfp4", [False, True])
def test_workload5_scheduled_equals_one_shot(mxfp4):
    """Workload 5 at full size: the per-step schedule, then the scheduled logits of the decode rows (paged pool)
    and the prefill rows (gathered chunk), equal the one-shot calls (checked against the oracle above) bit for
    bit.  The prefill rows' 32 chunks each are cut into segments at workgroup-share boundaries inside rows."""
    c = synth.workload(5)
    sbk, cbs, nd, rows = c["sbk"], c["cbs"], c["n_decode"], c["rows"]
    bs, nb = c["block_size"], c["num_blocks"]
    row = 68 if mxfp4 else ROW
    stride = bs * row
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    once = dsi.sparse_mqa_logits_mxfp4 if mxfp4 else dsi.sparse_mqa_logits
    ks_t, ke_t, cand_t = dev(c["ks"]), dev(c["ke"]), dev(c["cand"])
    si, end = dsi.expand_candidates(cand_t, ks_t, ke_t, cbs, sbk)
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    quant(dev(c["k_dec"]), dev(c["dec_slot_mapping"]), pool, bs, stride, nb)
    Lp = c["Lp"]
    pre = torch.zeros(Lp * row, dtype=torch.uint8, device="cuda")
    quant(dev(c["k_pre"]), dev(np.arange(Lp, dtype=np.int64)), pre, Lp, Lp * row, 1)
    q, w, bt, r2r = dev(c["q"]), dev(c["w"]), dev(c["block_table"]), dev(c["row_to_req"])
    paged = dict(block_table=bt, row_to_req=r2r, block_size=bs, block_stride_bytes=stride)
    sched_d = dsi.sparse_schedule(ks_t[:nd], ke_t[:nd], si[:nd], end[:nd], sbk, pool, num_k=nb, mxfp4=mxfp4, **paged)
    sched_p = dsi.sparse_schedule(ks_t[nd:], ke_t[nd:], si[nd:], end[nd:], sbk, pre, num_k=Lp, mxfp4=mxfp4)
    got_d = host(dsi.sparse_mqa_logits_scheduled(q[:nd], w[:nd], sched_d, sbk, pool, mxfp4=mxfp4))
    got_p = host(dsi.sparse_mqa_logits_scheduled(q[nd:], w[nd:], sched_p, sbk, pre, mxfp4=mxfp4))
    one_d = host(once(q[:nd], w[:nd], ks_t[:nd], ke_t[:nd], si[:nd], end[:nd], sbk, pool, num_k=nb, **paged))
    one_p = host(once(q[nd:], w[nd:], ks_t[nd:], ke_t[nd:], si[nd:], end[nd:], sbk, pre, num_k=Lp))
    assert np.array_equal(got_d, one_d), "decode rows"
    assert np.array_equal(got_p, one_p), "prefill rows"


def test_workload5_hierarchical_sparse():
    _sparse_workload(False)


def test_workload5_hierarchical_sparse_mxfp4():
    """Workload 5 on the MXFP4 cache (68-byte rows)."""
    _sparse_workload(True)


@pytest.mark.parametrize("L,bs", [(8192, 64), (131072, 128)])
def test_prefill_gather_full_size(L, bs):
    """The prefill chunk's history (8192 tokens of 64-token pages) and the longest hierarchical prefill
    request (131072 tokens of 128-token pages) gathered from a randomly permuted pool, whole output compared
    with the oracle's gather of the same pool bytes."""
    c = synth.gather_case(L, [L], bs)
    pool = np.random.default_rng(L).integers(0, 256, size=c["num_blocks"] * c["block_stride"], dtype=np.uint8)
    oracle.k_quant_and_cache(c["k"], c["slot_mapping"], pool, bs, c["block_stride"])
    ref = oracle.gather_prefill_k(pool, c["num_blocks"], bs, c["block_stride"], c["block_table"], c["cu"], L)
    got = host(dsi.gather_prefill_k(dev(pool), bs, dev(c["block_table"]), dev(c["cu"]), S=L))
    assert np.array_equal(got, ref)


def test_q_prep_full_chunk():
    """The 2048-token prefill chunk's q (64 heads x 128 dims) rotated, quantized and folded; every code and
    weight compared bit for bit with the oracle."""
    c = synth.q_prep_case(2, 2048, max_pos=8192)
    ref_q8, ref_w = oracle.q_rope_quant(c["q"], c["positions"], c["cos_sin"], c["w"], c["softmax_scale"],
                                        c["head_scale"])
    q8, w_out = dsi.q_rope_quant(dev(c["q"]), dev(c["positions"]), dev(c["cos_sin"]), dev(c["w"]),
                                 c["softmax_scale"], c["head_scale"])
    assert np.array_equal(host(q8), ref_q8)
    assert np.array_equal(host(w_out), ref_w)
