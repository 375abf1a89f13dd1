"""Pins for the oracle's integer index steps: candidate expansion, sparse-column remap and
request-local -> physical slot conversion (hand-derived golden cases plus properties the pages state)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", load("expand_cases.json")["cases"], ids=lambda c: c["name"])
def test_expand_golden(case):
    si, end = oracle.expand_candidates(np.array([case["cand"]], np.int32), np.array([case["ks"]], np.int32),
                                       np.array([case["ke"]], np.int32), case["cbs"], case["sbk"])
    assert si[0].tolist() == case["si"]
    assert int(end[0]) == case["end"]
    for c, pos in case["remap"]:
        got = oracle.topk_remap(np.array([[c]], np.int32), si, np.array([case["ks"]], np.int32), case["sbk"])
        assert int(got[0, 0]) == pos


@pytest.mark.parametrize("case", load("slot_cases.json")["cases"], ids=lambda c: c["name"])
def test_slot_golden(case):
    got = oracle.req_index_to_global_slot(np.array([case["p"]], np.int32), np.array([case["table"]], np.int32),
                                          case["block_size"], case["block_span"])
    assert got[0].tolist() == case["slot"]


def random_rows(rng, rows, K, sbk, ratio, aligned=True):
    cbs = sbk * ratio
    ks = (rng.integers(0, 20, rows) * (sbk if aligned else 1)).astype(np.int32)
    ke = (ks + rng.integers(0, 40 * sbk, rows)).astype(np.int32)
    ke[0] = ks[0]  # one empty row
    maxc = (np.maximum(ke - ks, 0) + cbs - 1) // cbs
    cand = np.empty((rows, K), np.int32)
    for r in range(rows):
        cand[r] = rng.integers(-3, int(maxc[r]) + 3, K)
    return cand, ks, ke, cbs


@pytest.mark.parametrize("sbk,ratio", [(16, 1), (8, 2), (128, 1), (64, 2)])
def test_expand_properties(sbk, ratio):
    rng = np.random.default_rng(30 + sbk + ratio)
    K = 32
    cand, ks, ke, cbs = random_rows(rng, 40, K, sbk, ratio)
    si, end = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    assert si.shape == (40, K * ratio)
    for r in range(40):
        base = ks[r] // sbk
        maxb = (max(ke[r] - ks[r], 0) + sbk - 1) // sbk
        flat = np.concatenate([cand[r] * ratio + j for j in range(ratio)]) if ratio > 1 else cand[r]
        valid = np.sort(flat[(flat >= 0) & (flat < maxb)])
        n = valid.size
        assert np.array_equal(si[r, :n] - base, valid)  # sorted, in range, duplicates kept
        assert np.all(si[r, n:] == (valid[-1] + base if n else base))  # tail repeats the last id
        assert 0 <= end[r] <= n * sbk
        if n:
            assert end[r] > (n - 1) * sbk
            last_tokens = min(max(int(ke[r]) - (int(valid[-1]) * sbk + int(ks[r])), 1), sbk)
            assert end[r] == (n - 1) * sbk + last_tokens
        # invariance under permuting the candidate row
        perm = rng.permutation(K)
        si2, end2 = oracle.expand_candidates(cand[r:r + 1, perm], ks[r:r + 1], ke[r:r + 1], cbs, sbk)
        assert np.array_equal(si2[0], si[r]) and end2[0] == end[r]


def test_expand_rejects_bad_ratio():
    with pytest.raises(ValueError):
        oracle.expand_candidates(np.zeros((1, 4), np.int32), np.zeros(1, np.int32), np.ones(1, np.int32), 48, 16)


def test_expand_strided_candidate_rows():
    rng = np.random.default_rng(31)
    cand, ks, ke, cbs = random_rows(rng, 8, 16, 16, 1)
    wide = np.full((8, 40), 12345, np.int32)
    wide[:, 7:23] = cand
    a = oracle.expand_candidates(wide[:, 7:23], ks, ke, cbs, 16)
    b = oracle.expand_candidates(cand, ks, ke, cbs, 16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("sbk,ratio", [(16, 1), (8, 2), (128, 1)])
def test_remap_covers_candidate_tokens(sbk, ratio):
    # for aligned ks: {remap(c) : c < end, token < ke} == multiset of candidate tokens in [0, ke - ks)
    rng = np.random.default_rng(40 + sbk)
    cand, ks, ke, cbs = random_rows(rng, 30, 16, sbk, ratio)
    si, end = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    W = si.shape[1] * sbk
    cols = np.tile(np.arange(W, dtype=np.int32), (30, 1))
    pos = oracle.topk_remap(cols, si, ks, sbk)
    for r in range(30):
        got = pos[r, :end[r]]
        got = np.sort(got[got < ke[r] - ks[r]])
        kv = max(int(ke[r] - ks[r]), 0)
        want = []
        maxc = (kv + cbs - 1) // cbs
        for c in cand[r]:
            if 0 <= c < maxc:
                want.extend(t for t in range(c * cbs, (c + 1) * cbs) if t < kv)
        assert np.array_equal(got, np.sort(np.array(want, dtype=np.int32)))


def test_remap_keeps_minus_one():
    si = np.array([[3, 5]], np.int32)
    got = oracle.topk_remap(np.array([[-1, 0, 17, -1]], np.int32), si, np.array([0], np.int32), 16)
    assert got.tolist() == [[-1, 48, 81, -1]]


def test_slot_identity_and_inverse_permutation():
    rng = np.random.default_rng(50)
    bs, nb = 64, 20
    p = rng.integers(-1, bs * nb, size=(3, 300)).astype(np.int32)
    ident = np.tile(np.arange(nb, dtype=np.int32), (3, 1))
    assert np.array_equal(oracle.req_index_to_global_slot(p, ident, bs, bs), p)
    perm = np.stack([rng.permutation(nb) for _ in range(3)]).astype(np.int32)
    slot = oracle.req_index_to_global_slot(p, perm, bs, bs)
    for r in range(3):
        inv = np.argsort(perm[r])
        v = slot[r] >= 0
        back = inv[slot[r][v] // bs] * bs + slot[r][v] % bs
        assert np.array_equal(back, p[r][v])
        assert np.all(slot[r][~v] == -1) and np.all(p[r][~v] < 0)


def test_slot_row_to_req():
    bt = np.array([[0, 1], [5, 6], [9, 8]], np.int32)
    p = np.array([[0, 70], [0, 70]], np.int32)
    got = oracle.req_index_to_global_slot(p, bt, 64, 64, row_to_req=np.array([2, 1], np.int32))
    assert got.tolist() == [[9 * 64, 8 * 64 + 6], [5 * 64, 6 * 64 + 6]]
