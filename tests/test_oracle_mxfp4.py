"""Pins for the oracle's MXFP4 indexer cache (FP4 E2M1 elements, one E8M0 scale per 32) and the sparse logits
on it.

Page "V4.1 indexer uses sparse MQA logits", motivation and implementation: the V4.1 sparse indexer runs on an
MXFP4 indexer cache and scores FP8 q against FP4 k.  The pages name the format only; it is the OCP Microscaling
format, whose element table, rounding and shared-scale rule are pinned here by hand-written values.  The logits
are pinned against the (separately pinned) FP8 path: keys representable in both formats give bit-identical
logits, and random keys agree with an fp64 recomputation.
"""
import numpy as np

import oracle
import synth

FP4 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_table_and_round_trip():
    want = FP4 + [-v for v in FP4]
    got = oracle.fp4_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got, np.array(want, np.float32))
    assert np.signbit(got[8])  # code 8 is -0
    assert np.array_equal(oracle.fp4_encode(got), np.arange(16, dtype=np.uint8))


def test_fp4_rounding_ties_and_saturation():
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,   # ties go to the even code
             0.26: 1, 0.3: 1, 1.3: 3, 2.6: 5, 4.9: 6, 5.1: 7,           # nearest
             6.0: 7, 7.0: 7, 1e6: 7, 0.1: 0}
    for x, c in cases.items():
        assert oracle.fp4_encode(np.float32(x)) == c, x
        assert oracle.fp4_encode(np.float32(-x)) == (c | 8), -x
    assert oracle.fp4_encode(np.float32(-0.1)) == 8  # rounds to -0


def _quant(rows_f32):
    kb = synth._bf16_bits(np.asarray(rows_f32, np.float32))
    n = kb.shape[0]
    pool = np.full(n * 68, 0xA5, np.uint8)
    oracle.k_quant_and_cache_mxfp4(kb, np.arange(n, dtype=np.int64), pool, n, n * 68)
    return pool.reshape(n, 68)


def _unpack(row):
    codes = np.empty(128, np.uint8)
    codes[0::2] = row[:64] & 15
    codes[1::2] = row[:64] >> 4
    return codes, row[64:68]


def test_zero_row_and_packing():
    r = _quant(np.zeros((1, 128)))[0]
    assert not r.any()  # codes 0, scale bytes 0 (2^-127)
    x = np.zeros(128, np.float32)
    x[0], x[1], x[5] = 0.5, -1.0, 6.0      # block 0: amax 6 -> shared exponent 0 -> scale byte 127
    x[32 + 3] = 3.0                          # block 1: amax 3 -> floor(log2 3) - 2 = -1 -> byte 126, 3 / 0.5 = 6
    x[64:96] = 0.0                           # block 2: zero
    x[96 + 31] = -0.25                       # block 3: amax 0.25 -> -4 -> byte 123, -0.25 * 16 = -4
    r = _quant(x[None])[0]
    assert r[0] == (0xA << 4 | 0x1) and r[2] == 0x70  # elements 0, 1 (-1.0 = code 8|2) and 5 (6.0, high nibble)
    assert list(r[64:68]) == [127, 126, 0, 123]
    codes, _ = _unpack(r)
    assert codes[35] == 7 and codes[127] == 8 | 6


def test_grid_rows_reproduce_and_saturation():
    rng = np.random.default_rng(61)
    for k in (-5, 0, 3):
        codes = rng.integers(0, 16, size=(4, 128)).astype(np.uint8)
        codes[:, ::32] = 7  # each block holds +6 * 2^k, which sets the scale
        x = oracle.fp4_decode(codes) * np.float32(2.0 ** k)
        r = _quant(x)
        got, sc = zip(*[_unpack(row) for row in r])
        got = np.stack(got)
        nz = oracle.fp4_decode(codes) != 0
        assert np.array_equal(got[nz], codes[nz]) and np.all(np.stack(sc) == 127 + k)
    # amax in [6, 8) * 2^k saturates to 6 * 2^k
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 1] = 7.0, 1.0
    codes, sc = _unpack(_quant(x)[0])
    assert codes[0] == 7 and codes[1] == 2 and sc[0] == 127


def _decode_mx(rows):
    out = np.empty((rows.shape[0], 128), np.float64)
    for i, row in enumerate(rows):
        codes, sc = _unpack(row)
        out[i] = np.array([FP4[c & 7] * (-1 if c & 8 else 1) for c in codes]) * 2.0 ** (np.repeat(sc, 32) - 127.0)
    return out


def test_quant_error_bound():
    rng = np.random.default_rng(62)
    x = synth._bf16_value(synth.draw_k(rng, 64)).astype(np.float64)
    dec = _decode_mx(_quant(x))
    for j in range(4):
        blk = x[:, 32 * j:32 * j + 32]
        se = np.floor(np.log2(np.abs(blk).max(axis=1))) - 2
        err = np.abs(dec[:, 32 * j:32 * j + 32] - blk)
        assert np.all(err <= 2.0 ** (se + 1)[:, None])          # half a step at the top (1) or saturation (< 2)
        small = np.abs(blk) < 6 * 2.0 ** se[:, None]
        assert np.all(err[small] <= 0.25 * np.maximum(np.abs(blk[small]), 2.0 ** se.repeat(32).reshape(-1, 32)[small]))


def _sparse_inputs(rng, rows, S, sbk=16, nsb=6):
    qf = synth.draw_q(rng, rows)
    q, w = synth.finish_q(rng, qf)
    si = np.sort(rng.integers(0, S // sbk, size=(rows, nsb)), axis=1).astype(np.int32)
    ks = np.zeros(rows, np.int32)
    ke = np.full(rows, S, np.int32)
    ke[0] = S - 5
    end = np.full(rows, nsb * sbk, np.int32)
    end[1] = nsb * sbk - 20
    return q, w, si, ks, ke, end


def test_logits_equal_fp8_path_on_keys_both_formats_hold():
    rng = np.random.default_rng(63)
    S, rows, sbk = 128, 3, 16
    codes = rng.integers(0, 16, size=(S, 128)).astype(np.uint8)
    codes[:, ::32] = 7
    kvals = oracle.fp4_decode(codes) * np.float32(2.0 ** -2)
    mx = _quant(kvals).reshape(-1)
    f8 = np.zeros((S, 132), np.uint8)
    f8[:, :128] = oracle.e4m3_encode(kvals)  # exact: fp4 values times 2^-2 are E4M3 values
    f8[:, 128:] = np.ones(S, np.float32).view(np.uint8).reshape(S, 4)
    assert np.array_equal(oracle.e4m3_decode(f8[:, :128]), kvals)
    q, w, si, ks, ke, end = _sparse_inputs(rng, rows, S, sbk)
    a = oracle.sparse_mqa_logits(q, w, ks, ke, si, end, sbk, f8.reshape(-1), out_f32=True)
    b = oracle.sparse_mqa_logits_mxfp4(q, w, ks, ke, si, end, sbk, mx, out_f32=True)
    assert np.array_equal(a, b)
    assert np.isinf(b[1, -20:]).all() and np.isfinite(b[2]).all()


def test_logits_against_fp64_paged():
    rng = np.random.default_rng(64)
    S, rows, sbk, bs = 256, 2, 16, 32
    k = synth.draw_k(rng, S)
    nb = S // bs + 2
    perm = rng.permutation(nb)[: S // bs].astype(np.int32)
    stride = bs * 68 + 16
    pool = np.zeros(nb * stride, np.uint8)
    slots = (perm[np.arange(S) // bs].astype(np.int64) * bs + np.arange(S) % bs)
    oracle.k_quant_and_cache_mxfp4(k, slots, pool, bs, stride)
    q, w, si, ks, ke, end = _sparse_inputs(rng, rows, S, sbk)
    bt = perm[None, :].repeat(rows, axis=0)
    got = oracle.sparse_mqa_logits_mxfp4(q, w, ks, ke, si, end, sbk, pool, block_table=bt, block_size=bs,
                                         block_stride=stride, out_f32=True)
    rowsmx = np.stack([pool[(s // bs) * 0 + perm[s // bs] * stride + (s % bs) * 68:][:68] for s in range(S)])
    kd = _decode_mx(rowsmx)
    qd = oracle.e4m3_decode(q).astype(np.float64)
    wd = synth._bf16_value(w).astype(np.float64)
    for r in range(rows):
        for c in range(si.shape[1] * sbk):
            tok = si[r, c // sbk] * sbk + c % sbk
            if c >= end[r] or tok >= ke[r]:
                assert got[r, c] == -np.inf
                continue
            terms = wd[r][:, None] * qd[r] * kd[tok][None, :]
            exact = terms.sum()
            assert abs(got[r, c] - exact) <= 2.0 ** -20 * np.abs(terms).sum() + 1e-30, (r, c)


def _paged_mx_pool(rng, k, bs, extra_pages=3, pad=16):
    """k rows [S, 128] (bf16 bits) MXFP4-quantized into a pool of permuted pages (stride bs*68 + pad)."""
    S = k.shape[0]
    npg = (S + bs - 1) // bs
    nb = npg + extra_pages
    perm = rng.permutation(nb)[:npg].astype(np.int32)
    stride = bs * 68 + pad
    pool = np.full(nb * stride, 0x5A, np.uint8)
    s = np.arange(S)
    oracle.k_quant_and_cache_mxfp4(k, perm[s // bs].astype(np.int64) * bs + s % bs, pool, bs, stride)
    return pool, perm, stride


def test_paged_decode_against_fp64():
    """O15 on ragged requests with two next-n rows each, permuted pages and padded page strides: every scored
    cell equals the fp64 sum of w*q*k over the independently decoded key (within fp32 accumulation), the
    row's last visible token is L - next_n + i, and everything past it (up to the output width) is -inf."""
    rng = np.random.default_rng(65)
    bs, next_n = 16, 2
    lens = np.array([37, 1, 70], np.int32)
    width = 80
    S = int(lens.max())
    k = synth.draw_k(rng, S)
    pool, perm, stride = _paged_mx_pool(rng, k, bs)
    B = lens.shape[0]
    bt = np.tile(perm, (B, 1))
    qf = synth.draw_q(rng, B * next_n)
    q, w = synth.finish_q(rng, qf)
    got = oracle.mqa_logits_paged_mxfp4(q, w, next_n, lens, pool, bs, stride, bt, width)
    rows = np.stack([pool[perm[s // bs] * stride + (s % bs) * 68:][:68] for s in range(S)])
    kd = _decode_mx(rows)
    qd = oracle.e4m3_decode(q).astype(np.float64)
    wd = synth._bf16_value(w).astype(np.float64)
    for b in range(B):
        for i in range(next_n):
            r = b * next_n + i
            ke = int(lens[b]) - next_n + i + 1
            assert np.all(got[r, max(ke, 0):] == -np.inf)
            for s in range(max(ke, 0)):
                terms = wd[r][:, None] * qd[r] * kd[s][None, :]
                assert abs(got[r, s] - terms.sum()) <= 2.0 ** -20 * np.abs(terms).sum() + 1e-30, (r, s)


def test_paged_decode_equals_fp8_path_on_keys_both_formats_hold():
    """Keys whose values are FP4 codes times 2^-2 in every 32-block (scale byte 125) are E4M3 values too:
    O15 on the MXFP4 pool and O2's paged decode on the FP8 pool (scale 1) give bit-identical logits."""
    rng = np.random.default_rng(66)
    bs, S = 32, 96
    codes = rng.integers(0, 16, size=(S, 128)).astype(np.uint8)
    codes[:, ::32] = 7  # every block reaches 6 * 2^-2, so its shared exponent is -2
    kvals = oracle.fp4_decode(codes) * np.float32(2.0 ** -2)
    kb = synth._bf16_bits(kvals)
    pool4, perm, stride4 = _paged_mx_pool(rng, kb, bs)
    stride8 = bs * 132
    pool8 = np.zeros(len(pool4) // stride4 * stride8, np.uint8)
    for s in range(S):
        row = pool8[perm[s // bs] * stride8 + (s % bs) * 132:][:132]
        row[:128] = oracle.e4m3_encode(kvals[s])
        row[128:] = np.ones(1, np.float32).view(np.uint8)
    lens = np.array([S, 50], np.int32)
    bt = np.tile(perm, (2, 1))
    q, w = synth.finish_q(rng, synth.draw_q(rng, 2))
    a = oracle.mqa_logits_paged(q, w, 1, lens, pool8, bs, stride8, bt, S)
    b = oracle.mqa_logits_paged_mxfp4(q, w, 1, lens, pool4, bs, stride4, bt, S)
    assert np.array_equal(a, b)
    assert np.isinf(b[1, 50:]).all() and np.isfinite(b[0]).all()
