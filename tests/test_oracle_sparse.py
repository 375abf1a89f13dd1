"""Pins for the oracle's sparse MQA logits and the hierarchical selection invariant.

vLLM PR 56254 summary: the consumer indexer scores only the candidate blocks and runs top-k in the
compressed space, then maps back to context positions; its tests check that the sparse path selects the
same values as dense logits masked to the candidates followed by top-k.
"""
import numpy as np
import pytest

import oracle
import synth


def gathered_rows(k_bf16):
    S = k_bf16.shape[0]
    rows = np.zeros((S, 132), np.uint8)
    oracle.k_quant_and_cache(k_bf16, np.arange(S), rows.reshape(-1), S, S * 132)
    return rows


def unique_candidates(rng, rows, ks, ke, cbs, K):
    cand = np.empty((rows, K), np.int32)
    for r in range(rows):
        m = (max(int(ke[r] - ks[r]), 0) + cbs - 1) // cbs
        ids = rng.choice(m, size=min(K, m), replace=False) if m else np.zeros(0, np.int64)
        row = np.concatenate([ids, np.full(K - ids.size, -1)]).astype(np.int32)
        rng.shuffle(row)
        cand[r] = row
    return cand


@pytest.mark.parametrize("sbk,ratio", [(16, 1), (8, 2), (32, 1)])
def test_sparse_selects_same_values_as_dense_masked(sbk, ratio):
    rng = np.random.default_rng(60 + sbk)
    cbs, S, T, K, k = sbk * ratio, 600, 6, 8, 40
    c = synth.prefill_case(61 + sbk, T=T, S=S, first_pos=S - T)
    rows = gathered_rows(c["k"])
    ks = np.array([0, 0, 0, sbk, 2 * sbk, 0], np.int32)  # aligned starts
    ke = c["ke"]
    cand = unique_candidates(rng, T, ks, ke, cbs, K)
    si, end = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    sp = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows, out_f32=True)
    col = oracle.topk_select(sp, np.full(T, sp.shape[1], np.int32), k)
    pos = oracle.topk_remap(col, si, ks, sbk)
    dense_idx, dense = oracle.dense_masked_topk(c["q"], c["w"], rows, ks, ke, cand, cbs, k)
    for r in range(T):
        v_sparse = np.sort(sp[r, col[r][col[r] >= 0]])
        v_dense = np.sort(dense[r, dense_idx[r][dense_idx[r] >= 0] + ks[r]])
        assert np.array_equal(v_sparse, v_dense)
        # the remapped positions score the same as the dense logits at those positions
        p = pos[r][pos[r] >= 0]
        assert np.array_equal(np.sort(dense[r, p + ks[r]]), v_dense)
        assert np.sum(pos[r] == -1) == np.sum(dense_idx[r] == -1)


def test_sparse_column_is_token_logit_rounded_once():
    rng = np.random.default_rng(70)
    sbk, S, T = 16, 300, 4
    c = synth.prefill_case(71, T=T, S=S, first_pos=S - T)
    rows = gathered_rows(c["k"])
    ks, ke = c["ks"], c["ke"]
    cand = np.array([[0, 5, 5, -1], [17, 3, 2, 1], [18, 18, 0, 9], [-1, -1, -1, -1]], np.int32)
    si, end = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    bf = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows)
    f32 = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows, out_f32=True)
    dense = oracle.mqa_logits_gathered(c["q"], c["w"], rows, ks, ke)
    for r in range(T):
        for col in range(si.shape[1] * sbk):
            tok = si[r, col // sbk] * sbk + col % sbk
            if col < end[r] and ks[r] <= tok < ke[r]:
                assert f32[r, col] == dense[r, tok]
                assert bf[r, col] == oracle.bf16_rne(np.array([dense[r, tok]], np.float32))[0]
            else:
                assert bf[r, col] == 0xFF80 and np.isneginf(f32[r, col])
    assert np.all(bf[3] == 0xFF80)  # no valid candidate: every column is -inf


def test_partial_block_duplicate_masked_by_token_range():
    # ke = 40, candidate 2 twice: columns of the duplicate block cover tokens 32..47, tokens >= 40 are -inf
    c = synth.prefill_case(72, T=1, S=48, first_pos=39)
    rows = gathered_rows(c["k"])
    si, end = oracle.expand_candidates(np.array([[2, 2, 0, -1]], np.int32), c["ks"], c["ke"], 16, 16)
    assert si[0].tolist() == [0, 2, 2, 2] and end[0] == 40
    f32 = oracle.sparse_mqa_logits(c["q"], c["w"], c["ks"], c["ke"], si, end, 16, rows, out_f32=True)
    assert np.all(np.isfinite(f32[0, :16])) and np.all(np.isfinite(f32[0, 16:24]))
    assert np.all(np.isneginf(f32[0, 24:32]))  # tokens 40..47
    assert np.all(np.isfinite(f32[0, 32:40])) and np.all(np.isneginf(f32[0, 40:]))


def test_paged_source_equals_gathered_source():
    rng = np.random.default_rng(73)
    sbk, bs = 16, 32
    c = synth.prefill_case(74, T=3, S=200, first_pos=197)
    rows = gathered_rows(c["k"])
    nblk = (200 + bs - 1) // bs
    perm = rng.permutation(nblk).astype(np.int32)
    stride = bs * 132
    pool = np.zeros(nblk * stride, np.uint8)
    for s in range(200):
        a = perm[s // bs] * stride + (s % bs) * 132
        pool[a:a + 132] = rows[s]
    ks, ke = np.zeros(3, np.int32), np.array([200, 150, 37], np.int32)
    cand = unique_candidates(rng, 3, ks, ke, sbk, 6)
    si, end = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    a = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows)
    b = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, pool,
                                 block_table=np.tile(perm, (2, 1)), row_to_req=np.array([1, 0, 1], np.int32),
                                 block_size=bs, block_stride=stride)
    assert np.array_equal(a, b)
