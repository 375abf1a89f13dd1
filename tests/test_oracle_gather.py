"""Pins for the oracle's prefill K gather.

Page "DeepSeek V3.2 sparse attention DSA inference flow", prefill/decode table: a prefill chunk collects the
history K of its requests out of the paged cache before scoring it (decode reads the cache in place).  Page
"V4.1 indexer uses sparse MQA logits", implementation breakdown: the indexer's forward chains that prefill K
gather with the paged decode path.

The pins do not restate the gather: (1) gathering a pool that k_quant_and_cache filled through a permuted
block table equals k_quant_and_cache writing the same k rows to consecutive slots of one contiguous block;
(2) hand-built cases with every row's source written out by hand; (3) an identity table over an unpacked
pool returns the pool's own bytes.
"""
import numpy as np

import oracle
import synth

ROW = 132


def _quantized_pool(c, fill=0x5A):
    pool = np.full(c["num_blocks"] * c["block_stride"], fill, dtype=np.uint8)
    oracle.k_quant_and_cache(c["k"], c["slot_mapping"], pool, c["block_size"], c["block_stride"])
    return pool


def _contiguous_rows(k):
    n = k.shape[0]
    rows = np.zeros(max(n, 1) * ROW, dtype=np.uint8)
    oracle.k_quant_and_cache(k, np.arange(n, dtype=np.int64), rows, max(n, 1), max(n, 1) * ROW)
    return rows.reshape(-1, ROW)[:n]


def test_gather_equals_contiguous_quantization():
    for seed, lens, bs, span in [(11, [37, 130, 1], 16, None), (12, [64, 64, 200], 64, 68), (13, [5], 8, 9),
                                 (14, [0, 17, 0, 33], 16, None)]:
        c = synth.gather_case(seed, lens, bs, span)
        pool = _quantized_pool(c)
        got = oracle.gather_prefill_k(pool, c["num_blocks"], bs, c["block_stride"], c["block_table"], c["cu"],
                                      c["S"])
        assert np.array_equal(got, _contiguous_rows(c["k"])), (seed, lens, bs, span)


def test_hand_case():
    # bs = 4, four pages; page p's token o is filled with the byte 16*p + o (scale bytes too).
    bs, nb = 4, 4
    pool = np.zeros((nb, bs, ROW), dtype=np.uint8)
    for p in range(nb):
        for o in range(bs):
            pool[p, o, :] = 16 * p + o
    bt = np.array([[2, 0, 3], [1, 7, 0]], dtype=np.int32)  # page 7 does not exist
    cu = np.array([0, 6, 9], dtype=np.int32)  # request 0: 6 tokens, request 1: 3 tokens
    got = oracle.gather_prefill_k(pool.ravel(), nb, bs, bs * ROW, bt, cu, 10)
    # request 0: tokens 0-3 on page 2, tokens 4-5 on page 0; request 1: tokens 0-2 on page 1; row 9 unowned
    expect = [0x20, 0x21, 0x22, 0x23, 0x00, 0x01, 0x10, 0x11, 0x12, None]
    for row, e in enumerate(expect):
        want = np.zeros(ROW, dtype=np.uint8) if e is None else np.full(ROW, e, dtype=np.uint8)
        assert np.array_equal(got[row], want), row
    # request 1 grows into its second block, whose page id 7 is outside the pool: zero rows
    got = oracle.gather_prefill_k(pool.ravel(), nb, bs, bs * ROW, bt, np.array([0, 6, 11], dtype=np.int32), 11)
    assert np.all(got[6:10] == np.array([0x10, 0x11, 0x12, 0x13], dtype=np.uint8)[:, None])
    assert np.all(got[10] == 0)
    # a narrower table (bt_width = 1) cuts request 0 after its first block
    got = oracle.gather_prefill_k(pool.ravel(), nb, bs, bs * ROW, bt, cu, 9, bt_width=1)
    assert np.all(got[4:6] == 0) and np.all(got[3] == 0x23) and np.all(got[6] == 0x10)


def test_offsets_and_truncation():
    c = synth.gather_case(15, [10, 7], 4)
    pool = _quantized_pool(c)
    ref = _contiguous_rows(c["k"])
    # cu starting at 3: three leading unowned rows, then the requests
    cu = c["cu"] + 3
    got = oracle.gather_prefill_k(pool, c["num_blocks"], 4, c["block_stride"], c["block_table"], cu, 22)
    assert np.all(got[:3] == 0) and np.array_equal(got[3:20], ref) and np.all(got[20:] == 0)
    # fewer output rows than tokens: the tail is cut
    got = oracle.gather_prefill_k(pool, c["num_blocks"], 4, c["block_stride"], c["block_table"], c["cu"], 12)
    assert np.array_equal(got, ref[:12])
    # an empty chunk
    got = oracle.gather_prefill_k(pool, c["num_blocks"], 4, c["block_stride"], c["block_table"],
                                  np.zeros(3, dtype=np.int32), 5)
    assert np.all(got == 0)


def test_identity_table_returns_pool_bytes():
    rng = np.random.default_rng(16)
    bs, nb = 16, 5
    pool = rng.integers(0, 256, size=nb * bs * ROW, dtype=np.uint8)
    bt = np.arange(nb, dtype=np.int32)[None, :]
    S = nb * bs - 3
    got = oracle.gather_prefill_k(pool, nb, bs, bs * ROW, bt, np.array([0, S], dtype=np.int32), S)
    assert np.array_equal(got.ravel(), pool[:S * ROW])
