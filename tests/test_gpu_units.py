"""GPU parity, one kernel at a time, against the oracle on identical input bytes.

Sizes are small enough for the oracle to finish in seconds but span several tiles and a ragged tail.
Integer and byte outputs must be bit-exact; logits use the tolerance rules in parity_util.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_amd as dsi
import synth
from parity_util import (ROW, assert_close, bf16_value, check_selection, dev, gathered_rows_oracle, host,
                         paged_pool_oracle, tol_bf16)

pytestmark = pytest.mark.gpu
K = 2048


# ----------------------------------------------------------------------------- k quant + cache insert
def test_k_quant_every_bf16_value_bit_exact():
    # amax = 448 makes the scale exactly 1, so every bf16 value in [-448, 448] is encoded as itself:
    # an exhaustive check of the device rounding (ties, subnormals, saturation edge).
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    vals = x[np.isfinite(x) & (np.abs(x) <= 448)]
    n = (vals.size + 126) // 127
    k = np.zeros((n, 128), np.float32)
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    k[:, :127] = flat.reshape(n, 127)
    k[:, 127] = 448.0
    kb = synth._bf16_bits(k)
    bs, stride = 16, 16 * ROW
    nb = (n + bs - 1) // bs
    slots = np.arange(n, dtype=np.int64)
    ref = paged_pool_oracle(kb, slots, nb, bs, stride)
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache(dev(kb), dev(slots), pool, bs, stride, nb)
    assert np.array_equal(host(pool), ref)


@pytest.mark.parametrize("n,bs,extra", [(1, 16, 0), (1000, 64, 16), (4099, 128, 48)])
def test_k_quant_random_rows_packed_pool(n, bs, extra):
    rng = np.random.default_rng(n)
    kb = synth.draw_k(rng, n)
    kb[: min(n, 3)] = synth._bf16_bits(rng.standard_normal((min(n, 3), 128)).astype(np.float32) * 1e-6)  # tiny
    if n > 5:
        kb[4] = 0
    stride = bs * ROW + extra
    nb = (n + bs - 1) // bs + 2
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[::7] = -1  # padding tokens
    ref = paged_pool_oracle(kb, slots, nb, bs, stride)
    # the kernel only writes the rows of valid slots: start both from the same sentinel
    ref_s = np.full_like(ref, 0xA5)
    written = np.zeros(ref.size, bool)
    for s in slots[slots >= 0]:
        a = (s // bs) * stride + (s % bs) * ROW
        written[a:a + ROW] = True
    ref_s[written] = ref[written]
    pool = torch.full((nb * stride,), 0xA5, dtype=torch.uint8, device="cuda")
    wide = np.zeros((n, 160), np.uint16)
    wide[:, :128] = kb
    dsi.k_quant_and_cache(dev(wide)[:, :128], dev(slots), pool, bs, stride, nb)
    assert np.array_equal(host(pool), ref_s)


# ----------------------------------------------------------------------------- dense prefill logits
def _exact_int_inputs(rng, T, S):
    table = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E, 8: 0x50}
    enc = np.vectorize(lambda v: table[abs(int(v))] | (0x80 if v < 0 else 0))
    q = enc(rng.integers(-8, 9, size=(T, 64, 128))).astype(np.uint8)
    rows = np.zeros((S, ROW), np.uint8)
    rows[:, :128] = enc(rng.integers(-8, 9, size=(S, 128))).astype(np.uint8)
    rows[:, 128:] = np.ones(S, np.float32).view(np.uint8).reshape(S, 4)
    w = synth._bf16_bits((rng.choice([-1.0, 1.0], (T, 64)) * 2.0 ** rng.integers(-3, 4, (T, 64))).astype(np.float32))
    return q, w, rows


def test_prefill_exact_integer_bit_exact():
    rng = np.random.default_rng(100)
    T, S = 19, 333
    q, w, rows = _exact_int_inputs(rng, T, S)
    ks = np.zeros(T, np.int32)
    ke = np.full(T, S, np.int32)
    ref = oracle.mqa_logits_gathered(q, w, rows, ks, ke)
    out = dsi.mqa_logits_prefill(dev(q), dev(w), dev(rows), dev(ks), dev(ke))
    assert np.array_equal(host(out), ref)


def test_prefill_subnormal_codes_bit_exact():
    # q codes drawn from the E4M3 subnormals (m * 2^-9) and zero, k small integers, unit scales and
    # power-of-two weights: every partial sum is exact, so the device decode of subnormals must be exact
    rng = np.random.default_rng(101)
    T, S = 9, 200
    q, w, rows = _exact_int_inputs(rng, T, S)
    sub = np.array([0x00, 0x01, 0x02, 0x03, 0x04, 0x05, 0x06, 0x07, 0x81, 0x82, 0x83, 0x84, 0x85, 0x86, 0x87], np.uint8)
    q = sub[rng.integers(0, sub.size, size=q.shape)]
    ks, ke = np.zeros(T, np.int32), np.full(T, S, np.int32)
    ref = oracle.mqa_logits_gathered(q, w, rows, ks, ke)
    out = dsi.mqa_logits_prefill(dev(q), dev(w), dev(rows), dev(ks), dev(ke))
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("T,S,seed", [(37, 1001, 1), (8, 3072, 2), (5, 64, 3), (16, 1027, 4)])
def test_prefill_ragged_ranges_and_guards(T, S, seed):
    rng = np.random.default_rng(seed)
    c = synth.prefill_case(seed, T=T, S=S, first_pos=max(S - T, 0))
    rows = gathered_rows_oracle(c["k"])
    ks = rng.integers(0, S, T).astype(np.int32)
    ke = (ks + rng.integers(-5, S, T)).astype(np.int32)
    ks[0], ke[0] = 0, S + 50  # ke beyond S is clipped
    ks[1], ke[1] = 10, 10 if T > 1 else ke[1]  # empty row
    ref = oracle.mqa_logits_gathered(c["q"], c["w"], rows, ks, np.minimum(ke, S))
    ld = S + 13
    out = torch.full((T, ld), 7.25, dtype=torch.float32, device="cuda")
    dsi.mqa_logits_prefill(dev(c["q"]), dev(c["w"]), dev(rows), dev(ks), dev(ke), out=out[:, :S])
    got = host(out)
    valid = np.isfinite(ref)
    assert_close(got[:, :S][valid], ref[valid])
    assert np.all(got[:, :S][~valid] == 7.25), "entries outside [ks, ke) must stay untouched"
    assert np.all(got[:, S:] == 7.25)


def test_prefill_uses_the_k_scale_per_row():
    # same codes, per-row scales of 2^j: logits scale exactly with the row scale
    rng = np.random.default_rng(5)
    c = synth.prefill_case(6, T=4, S=96, first_pos=92)
    rows = gathered_rows_oracle(c["k"])
    ks, ke = np.zeros(4, np.int32), np.full(4, 96, np.int32)
    base = host(dsi.mqa_logits_prefill(dev(c["q"]), dev(c["w"]), dev(rows), dev(ks), dev(ke)))
    rows2 = rows.copy()
    sc = rows2[:, 128:].copy().view(np.float32)[:, 0] * (2.0 ** (np.arange(96) % 5)).astype(np.float32)
    rows2[:, 128:] = sc.astype(np.float32).view(np.uint8).reshape(96, 4)
    got = host(dsi.mqa_logits_prefill(dev(c["q"]), dev(c["w"]), dev(rows2), dev(ks), dev(ke)))
    assert np.array_equal(got, base * (2.0 ** (np.arange(96) % 5)).astype(np.float32)[None, :])


# ----------------------------------------------------------------------------- paged decode logits
@pytest.mark.parametrize("next_n,bs,extra,long", [(1, 64, 0, False), (2, 64, 16, False), (3, 16, 0, False),
                                                   (4, 32, 32, False), (1, 64, 0, True), (2, 16, 0, True),
                                                   (4, 64, 16, True)])
def test_decode_parity_ragged(next_n, bs, extra, long):
    """Short ragged lengths, and long ones that span many 256-key chunks and several jobs per
    request (the double-buffered gather alternates buffers across job boundaries)."""
    lens = [4099, 2048 * 8 + 1, 2048 * 8, 2048 * 3 + 257, 9000] if long else [1, 15, 16, 17, 300, 1000 + next_n, 2049]
    c = synth.decode_case(10 + next_n, B=len(lens), next_n=next_n, lmin=0, lmax=0, block_size=bs, lens=lens)
    stride = bs * ROW + extra
    nb = c["num_blocks"]
    pool_np = paged_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    width = max(lens) + 3
    ref = oracle.mqa_logits_paged(c["q"], c["w"], next_n, c["context_lens"], pool_np, bs, stride,
                                  c["block_table"], width)
    ld = width + 5
    out = torch.full((len(lens) * next_n, ld), -3.5, dtype=torch.float32, device="cuda")
    dsi.paged_mqa_logits_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_np), bs,
                                dev(c["block_table"]), width, next_n=next_n, out=out[:, :width],
                                block_stride_bytes=stride, num_blocks=nb)
    got = host(out)
    valid = np.isfinite(ref)
    assert_close(got[:, :width][valid], ref[valid])
    assert np.all(got[:, :width][~valid] == -3.5) and np.all(got[:, width:] == -3.5)


def test_decode_bad_page_ids_score_minus_inf():
    c = synth.decode_case(20, B=2, next_n=1, lmin=0, lmax=0, block_size=16, lens=[64, 64])
    bs, stride, nb = 16, 16 * ROW, c["num_blocks"]
    pool_np = paged_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    bt = c["block_table"].copy()
    bt[0, 1] = nb + 100  # out of range page
    bt[1, 2] = -7
    out = dsi.paged_mqa_logits_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_np), bs, dev(bt),
                                      64, block_stride_bytes=stride, num_blocks=nb)
    got = host(out)
    assert np.all(np.isneginf(got[0, 16:32])) and np.all(np.isneginf(got[1, 32:48]))
    ref = oracle.mqa_logits_paged(c["q"], c["w"], 1, c["context_lens"], pool_np, bs, stride, c["block_table"], 64)
    keep = np.ones((2, 64), bool)
    keep[0, 16:32] = False
    keep[1, 32:48] = False
    assert_close(got[keep], ref[keep])


# ----------------------------------------------------------------------------- top-k
def _rows_with_ties(rng, rows, width):
    x = (rng.standard_normal((rows, width)) * 50).astype(np.float32)
    x[:, ::3] = np.round(x[:, ::3])
    x[0, :] = 1.5  # all equal
    return x


@pytest.mark.parametrize("width,k", [(3000, 2048), (2048, 2048), (2049, 2048), (700, 2048), (8192, 2048),
                                     (100, 7), (8193, 2048), (16384, 1000), (40000, 2048)])
def test_topk_f32_same_input_exact_values(width, k):
    rng = np.random.default_rng(width + k)
    rows = 8
    x = _rows_with_ties(rng, rows, width)
    x[1, 5] = np.nan
    x[1, 6] = np.inf
    x[2, 7] = -np.inf
    x[3, :] = 0.0
    x[3, ::2] = -0.0
    # Adjacent floats 1 + i*2^-23 share every key bit but the lowest ones, so the last
    # resolution digit decides the boundary.  Row 6: up to 5000 of them (a boundary bin
    # larger than the in-LDS candidate list); row 7: 1000 of them under 1500 larger values
    # (a boundary bin of 1000 columns resolved in LDS).
    adj = lambda n: rng.permutation(np.float32(1.0) + np.arange(n, dtype=np.float32) * np.float32(2.0 ** -23))
    n6 = min(width, 5000)
    x[6, :n6] = adj(n6)
    if width >= 2500:
        x[7, :] = rng.uniform(-1.0, 0.5, width).astype(np.float32)
        x[7, :1000] = adj(1000)
        x[7, 1000:2500] = rng.uniform(2.0, 3.0, 1500).astype(np.float32)
        x[7] = rng.permutation(x[7])
    starts = rng.integers(0, max(width // 4, 1), rows).astype(np.int32)
    ends = np.minimum(starts + rng.integers(0, width, rows), width).astype(np.int32)
    ends[0] = width
    starts[0] = 0
    starts[6:] = 0
    ends[6:] = width
    ref = oracle.topk_select(x, ends, k, starts=starts)
    got = host(dsi.topk_select(dev(x), dev(ends), k=k, row_starts=dev(starts)))
    for r in range(rows):
        check_selection(got[r], ref[r], x[r], rule="exact", start=starts[r], end=ends[r])
        g = got[r][got[r] >= 0] + starts[r]
        o = ref[r][ref[r] >= 0] + starts[r]
        assert np.array_equal(np.sort(x[r, g]), np.sort(x[r, o]))


@pytest.mark.parametrize("width", [8192, 16384])
def test_topk_bf16_exact_values(width):
    rng = np.random.default_rng(7)
    vals = (rng.standard_normal((9, width)) * 8).astype(np.float32)
    bits = synth._bf16_bits(vals)
    bits[1, :4000] = 0xFF80
    bits[2, :] = 0xFF80
    bits[6, :] = 0x4000  # one value everywhere: the boundary bin outgrows the candidate list
    ends = np.array([width, width, width, 100, 2048, 2047, width, 5000, 0], np.int32)
    ref = oracle.topk_select(bits, ends, 2048, bf16=True)
    got = host(dsi.topk_select(dev(bits), dev(ends), k=2048))
    f = bf16_value(bits)
    for r in range(9):
        check_selection(got[r], ref[r], f[r], rule="exact", end=ends[r])
        assert np.array_equal(np.sort(f[r, got[r][got[r] >= 0]]), np.sort(f[r, ref[r][ref[r] >= 0]]))


@pytest.mark.parametrize("bf16", [False, True])
def test_topk_many_long_rows(bf16):
    """Enough long rows to fill the CUs (520 rows of 20000 columns): one 1024-thread workgroup per row, reading the
    row twice; ordinary rows, heavy ties (the boundary bin larger than the candidate list, resolved by passes over
    the row), rows with fewer than k finite values, ragged starts and ends; selected values against the oracle's."""
    rng = np.random.default_rng(53 + bf16)
    rows, width = 520, 20000
    x = (rng.standard_normal((rows, width)) * 20).astype(np.float32)
    x[1, :] = 3.0
    x[2, 500:] = -np.inf
    x[3] = np.round(x[3])
    x[4, ::3] = 9.5
    ends = rng.integers(15000, width + 1, rows).astype(np.int32)
    starts = rng.integers(0, 3000, rows).astype(np.int32)
    ends[:5], starts[:5] = width, 0
    if bf16:
        bits = synth._bf16_bits(x)
        vals = bf16_value(bits)
        ref = oracle.topk_select(bits, ends, 2048, starts=starts, bf16=True)
        got = host(dsi.topk_select(dev(bits), dev(ends), k=2048, row_starts=dev(starts)))
    else:
        vals = x
        ref = oracle.topk_select(x, ends, 2048, starts=starts)
        got = host(dsi.topk_select(dev(x), dev(ends), k=2048, row_starts=dev(starts)))
    for r in range(rows):
        check_selection(got[r], ref[r], vals[r], rule="exact", start=starts[r], end=ends[r])
        g = got[r][got[r] >= 0] + starts[r]
        o = ref[r][ref[r] >= 0] + starts[r]
        assert np.array_equal(np.sort(vals[r, g]), np.sort(vals[r, o]))
    assert np.sum(got[2] >= 0) == 500


@pytest.mark.parametrize("bf16,rows", [(False, 8), (True, 8), (False, 13)])
def test_topk_split_long_rows(bf16, rows):
    """Few long rows are split between workgroups; cover the take-all, all-invalid, heavy-tie
    (boundary bin larger than the candidate list) and ordinary rows, and a row count that leaves
    some of the workgroup numbers (a row's slices share one XCD) without a row."""
    rng = np.random.default_rng(21 + bf16)
    width = 50000
    x = (rng.standard_normal((rows, width)) * 40).astype(np.float32)
    x[1, 1000:] = -np.inf           # 1000 valid: take all, pad with -1
    x[2, :] = np.nan                # nothing valid
    x[3, :] = 2.5                   # one value everywhere
    x[4, ::2] = 7.0                 # a heavy tie inside the top 2048
    x[5] = np.round(x[5] / 8) * 8   # many ties
    ends = np.array([width, width, width, width, width, 30001, 20000, 49999], np.int32)
    starts = np.array([0, 0, 0, 0, 3, 17, 0, 12345], np.int32)
    ends = np.concatenate([ends, rng.integers(20000, width + 1, rows - 8)]).astype(np.int32)
    starts = np.concatenate([starts, rng.integers(0, 5000, rows - 8)]).astype(np.int32)
    if bf16:
        bits = synth._bf16_bits(x)
        vals = bf16_value(bits)
        ref = oracle.topk_select(bits, ends, 2048, starts=starts, bf16=True)
        got = host(dsi.topk_select(dev(bits), dev(ends), k=2048, row_starts=dev(starts)))
    else:
        vals = x
        ref = oracle.topk_select(x, ends, 2048, starts=starts)
        got = host(dsi.topk_select(dev(x), dev(ends), k=2048, row_starts=dev(starts)))
    for r in range(rows):
        check_selection(got[r], ref[r], vals[r], rule="exact", start=starts[r], end=ends[r])
        g = got[r][got[r] >= 0] + starts[r]
        o = ref[r][ref[r] >= 0] + starts[r]
        assert np.array_equal(np.sort(vals[r, g]), np.sort(vals[r, o]))
    assert np.all(got[2] == -1) and np.sum(got[1] >= 0) == 1000


def test_topk_strided_rows_and_out():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((4, 5000)) * 3).astype(np.float32)
    big = torch.zeros((4, 6000), dtype=torch.float32, device="cuda")
    big[:, 100:5100] = dev(x)
    out = torch.full((4, 2100), -9, dtype=torch.int32, device="cuda")
    ends = np.full(4, 5000, np.int32)
    dsi.topk_select(big[:, 100:5100], dev(ends), k=2048, out=out[:, 10:2058], max_width=5000)
    got = host(out)
    assert np.all(got[:, :10] == -9) and np.all(got[:, 2058:] == -9)
    ref = oracle.topk_select(x, ends, 2048)
    for r in range(4):
        check_selection(got[r, 10:2058], ref[r], x[r], rule="exact")


# ----------------------------------------------------------------------------- expansion / remap / slot
@pytest.mark.parametrize("sbk,ratio,K", [(16, 1, 4), (8, 2, 16), (128, 1, 64), (64, 2, 256), (32, 1, 512)])
def test_expand_bit_exact(sbk, ratio, K):
    rng = np.random.default_rng(sbk * 7 + K)
    rows, cbs = 300, sbk * ratio
    ks = (rng.integers(0, 30, rows) * sbk).astype(np.int32)
    ks[::5] += rng.integers(0, sbk, ks[::5].size).astype(np.int32)  # unaligned starts too
    ke = (ks + rng.integers(-10, 60 * cbs, rows)).astype(np.int32)
    maxc = (np.maximum(ke - ks, 0) + cbs - 1) // cbs
    cand = np.stack([rng.integers(-2, int(m) + 3, K) for m in maxc]).astype(np.int32)
    cand[::3, : K // 2] = cand[::3, K // 2:K // 2 * 2]  # duplicates
    si_ref, end_ref = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    wide = np.full((rows, K + 9), 555, np.int32)
    wide[:, 3:3 + K] = cand
    ks2 = np.zeros((rows, 2), np.int32)
    ks2[:, 1] = ks
    si, end = dsi.expand_candidates(dev(wide)[:, 3:3 + K], dev(ks2)[:, 1], dev(ke), cbs, sbk)
    assert np.array_equal(host(si), si_ref) and np.array_equal(host(end), end_ref)


def test_expand_golden_cases():
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "expand_cases.json")))["cases"]
    for c in cases:
        si, end = dsi.expand_candidates(dev(np.array([c["cand"]], np.int32)), dev(np.array([c["ks"]], np.int32)),
                                        dev(np.array([c["ke"]], np.int32)), c["cbs"], c["sbk"])
        assert host(si)[0].tolist() == c["si"] and int(host(end)[0]) == c["end"], c["name"]


def test_remap_bit_exact_and_alias():
    rng = np.random.default_rng(9)
    rows, nsb, sbk, k = 50, 64, 128, 2048
    si = np.sort(rng.integers(0, 1000, (rows, nsb)), axis=1).astype(np.int32)
    ks = (rng.integers(0, 8, rows) * sbk).astype(np.int32)
    col = rng.integers(-1, nsb * sbk, (rows, k)).astype(np.int32)
    ref = oracle.topk_remap(col, si, ks, sbk)
    got = host(dsi.topk_remap(dev(col), dev(si), dev(ks), sbk))
    assert np.array_equal(got, ref)
    t = dev(col)
    dsi.topk_remap(t, dev(si), dev(ks), sbk, out=t)  # in place
    assert np.array_equal(host(t), ref)


def test_slot_bit_exact_packed_and_alias():
    import json
    import os
    rng = np.random.default_rng(10)
    rows, k, bs, nreq = 40, 2048, 64, 7
    bt = np.stack([rng.permutation(2000)[:1100] for _ in range(nreq)]).astype(np.int32)
    r2r = rng.integers(0, nreq, rows).astype(np.int32)
    idx = rng.integers(-1, 1100 * bs, (rows, k)).astype(np.int32)
    for span in (64, 68):
        ref = oracle.req_index_to_global_slot(idx, bt, bs, span, row_to_req=r2r)
        got = host(dsi.req_index_to_global_slot(dev(idx), dev(bt), bs, span, row_to_req=dev(r2r)))
        assert np.array_equal(got, ref)
    t = dev(idx)
    dsi.req_index_to_global_slot(t, dev(bt), bs, 64, row_to_req=dev(r2r), out=t)
    assert np.array_equal(host(t), oracle.req_index_to_global_slot(idx, bt, bs, 64, row_to_req=r2r))
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "slot_cases.json")))["cases"]
    for c in cases:
        got = host(dsi.req_index_to_global_slot(dev(np.array([c["p"]], np.int32)),
                                                dev(np.array([c["table"]], np.int32)), c["block_size"],
                                                c["block_span"]))
        assert got[0].tolist() == c["slot"], c["name"]


# ----------------------------------------------------------------------------- sparse MQA logits
@pytest.mark.parametrize("sbk,ratio", [(128, 1), (16, 1), (8, 2), (32, 2)])
def test_sparse_gathered_parity(sbk, ratio):
    rng = np.random.default_rng(sbk + ratio)
    cbs, S, T, K = sbk * ratio, 3001, 12, 16
    c = synth.prefill_case(30 + sbk, T=T, S=S, first_pos=S - T)
    rows = gathered_rows_oracle(c["k"])
    ks = np.zeros(T, np.int32)
    ks[3] = sbk * 2
    ke = c["ke"].copy()
    ke[5] = 40
    maxb = (np.maximum(ke - ks, 0) + cbs - 1) // cbs
    cand = synth.draw_candidates(rng, maxb, num=K, distinct=min(12, int(maxb.min())), dup=2)
    si, end = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    ref_bits = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows)
    ref_f32 = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, rows, out_f32=True)
    got = host(dsi.sparse_mqa_logits(dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(si), dev(end), sbk, dev(rows)))
    valid = np.isfinite(ref_f32)
    assert np.array_equal(got[~valid], ref_bits[~valid])  # same -inf pattern
    assert_close(bf16_value(got[valid]), ref_f32[valid], tol_fn=tol_bf16, what="sparse logits")


@pytest.mark.parametrize("sbk,bs", [(128, 128), (16, 64), (8, 16)])
def test_sparse_paged_parity(sbk, bs):
    rng = np.random.default_rng(sbk * 3 + bs)
    lens = [700, 1, 129, 3000, 2048]
    c = synth.decode_case(40 + sbk, B=len(lens), next_n=1, lmin=0, lmax=0, block_size=bs, lens=lens)
    stride, nb = bs * ROW, c["num_blocks"]
    pool_np = paged_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    rows = len(lens)
    ks = np.zeros(rows, np.int32)
    ke = np.array(lens, np.int32)
    maxb = (np.maximum(ke - ks, 0) + sbk - 1) // sbk
    cand = synth.draw_candidates(rng, maxb, num=8, distinct=6, dup=1)
    si, end = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    r2r = np.arange(rows, dtype=np.int32)
    ref_f32 = oracle.sparse_mqa_logits(c["q"], c["w"], ks, ke, si, end, sbk, pool_np, block_table=c["block_table"],
                                       row_to_req=r2r, block_size=bs, block_stride=stride, out_f32=True)
    got = host(dsi.sparse_mqa_logits(dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(si), dev(end), sbk,
                                     dev(pool_np), block_table=dev(c["block_table"]), row_to_req=dev(r2r),
                                     block_size=bs, block_stride_bytes=stride, num_k=nb))
    valid = np.isfinite(ref_f32)
    assert np.all(got[~valid] == 0xFF80)
    assert_close(bf16_value(got[valid]), ref_f32[valid], tol_fn=tol_bf16, what="sparse paged logits")


# ----------------------------------------------------------------------------- prefill K gather
def _gather_inputs(seed, lens, bs, span=None):
    c = synth.gather_case(seed, lens, bs, span)
    rng = np.random.default_rng(seed + 1000)
    pool = rng.integers(0, 256, size=c["num_blocks"] * c["block_stride"], dtype=np.uint8)  # garbage elsewhere
    oracle.k_quant_and_cache(c["k"], c["slot_mapping"], pool, bs, c["block_stride"])
    return c, pool


def _gather_both(c, pool, bs, bt, cu, S, bt_width=None, extra_rows=5):
    ref = oracle.gather_prefill_k(pool, c["num_blocks"], bs, c["block_stride"], bt, cu, S, bt_width=bt_width)
    out = torch.full(((S + extra_rows) * ROW,), 0xEE, dtype=torch.uint8, device="cuda")
    dsi.gather_prefill_k(dev(pool), bs, dev(bt), dev(cu), S=S, out=out, block_stride_bytes=c["block_stride"],
                         num_blocks=c["num_blocks"], bt_width=bt_width)
    got = host(out)
    assert np.all(got[S * ROW:] == 0xEE), "wrote past row S"
    return got[:S * ROW].reshape(S, ROW), ref


@pytest.mark.parametrize("lens,bs,span", [([37, 130, 1], 16, None), ([64, 64, 200], 64, 68), ([5], 8, 9),
                                          ([0, 17, 0, 33], 16, None), ([3000, 1, 8191, 777], 64, None),
                                          ([301, 250], 6, 7), ([129, 4, 128], 128, None)])
def test_gather_bit_exact(lens, bs, span):
    c, pool = _gather_inputs(sum(lens) + bs, lens, bs, span)
    got, ref = _gather_both(c, pool, bs, c["block_table"], c["cu"], c["S"])
    assert np.array_equal(got, ref)
    # and it is exactly the contiguous quantization of the same k rows
    assert np.array_equal(got, gathered_rows_oracle(c["k"]))


def test_gather_missing_pages_offsets_and_truncation():
    lens, bs = [100, 45, 260], 16
    c, pool = _gather_inputs(77, lens, bs)
    bt = c["block_table"].copy()
    bt[0, 2] = -1                      # missing page
    bt[1, 1] = c["num_blocks"] + 3     # page beyond the pool
    bt[2, 5] = c["num_blocks"]
    got, ref = _gather_both(c, pool, bs, bt, c["cu"], c["S"])
    assert np.array_equal(got, ref) and np.all(got[32:48] == 0)
    # a narrower table, a chunk that starts at row 7, an output longer and one shorter than the chunk
    for cu, S, width in [(c["cu"], c["S"], 3), (c["cu"] + 7, c["S"] + 20, None), (c["cu"], 150, None),
                         (c["cu"] + 1, 3, None)]:
        got, ref = _gather_both(c, pool, bs, bt, cu, S, bt_width=width)
        assert np.array_equal(got, ref), (S, width)
    # no requests: every row is zero
    got, ref = _gather_both(c, pool, bs, bt, np.zeros(1, dtype=np.int32), 9)
    assert np.array_equal(got, ref) and not got.any()


# ----------------------------------------------------------------------------- q RoPE + quant + weight fold
@pytest.mark.parametrize("interleave", [False, True])
def test_q_rope_quant_bit_exact_strided(interleave):
    T, max_pos = 37, 4096
    c = synth.q_prep_case(31 + interleave, T, max_pos=max_pos)
    q, pos, w = c["q"].copy(), c["positions"].copy(), c["w"]
    pos[3], pos[7] = -1, max_pos          # outside the table: zero rows
    q[5, 9] = 0                           # an all-zero head row: scale 1e-4/448
    q[6, 2] = synth._bf16_bits(synth._bf16_value(q[6, 2]) * np.float32(1e-30))  # tiny values
    ref_q8, ref_w = oracle.q_rope_quant(q, pos, c["cos_sin"], w, c["softmax_scale"], c["head_scale"], interleave)
    # q as a column slice of a wider projection output, w as a slice of [T, 192]
    q_wide = np.zeros((T, 64 * 128 + 64), np.uint16)
    q_wide[:, :8192] = q.reshape(T, -1)
    w_wide = np.zeros((T, 192), np.uint16)
    w_wide[:, 128:] = w
    qt, wt = dev(q_wide), dev(w_wide)
    q8, w_out = dsi.q_rope_quant(qt[:, :8192], dev(pos), dev(c["cos_sin"]), wt[:, 128:], c["softmax_scale"],
                                 c["head_scale"], interleave=interleave)
    assert np.array_equal(host(q8), ref_q8)
    assert np.array_equal(host(w_out), ref_w)


# ----------------------------------------------------------------------------- context-parallel top-k
def test_topk_values_bit_exact():
    rng = np.random.default_rng(51)
    rows, W, k = 5, 3000, 300
    logits = rng.standard_normal((rows, W)).astype(np.float32)
    starts = np.array([0, 100, 2999, 5, 1000], np.int32)
    idx = rng.integers(-1, 2100, size=(rows, k)).astype(np.int32)  # some past max_width from their start
    ref_v, ref_g = oracle.topk_values(logits, idx, starts=starts, index_scale=3, index_offset=7, max_width=2900)
    v, g = dsi.topk_values(dev(logits), dev(idx), row_starts=dev(starts), index_scale=3, index_offset=7,
                           max_width=2900)
    assert np.array_equal(host(v), ref_v) and np.array_equal(host(g), ref_g)


def _candidate_lists(rng, rows, W, R, k, kind):
    """Oracle-made candidate lists of R contiguous slices of random rows."""
    x = rng.standard_normal((rows, W)).astype(np.float32)
    if kind == "ties":
        x = (np.round(x * 2) / 2).astype(np.float32)
    elif kind == "nonfinite":
        m = rng.random((rows, W))
        x[m < 0.05] = np.inf
        x[(m >= 0.05) & (m < 0.1)] = np.nan
    ends = rng.integers(W // 2, W + 1, size=rows).astype(np.int32)
    ends[0] = 3  # fewer valid values than k
    bounds = np.linspace(0, W, R + 1).astype(np.int32)
    vals, gidx = [], []
    for r in range(R):
        lo, hi = int(bounds[r]), int(bounds[r + 1])
        st = np.full(rows, lo, np.int32)
        idx = oracle.topk_select(x, np.minimum(ends, hi).astype(np.int32), k, starts=st)
        v, g = oracle.topk_values(x, idx, starts=st, index_offset=lo)
        vals.append(v)
        gidx.append(g)
    return x, ends, np.stack(vals), np.stack(gidx)


def _check_merge(got, ref, vals, gidx):
    for r in range(got.shape[0]):
        cand = {}
        for v, g in zip(vals[:, r].ravel(), gidx[:, r].ravel()):
            if g >= 0 and np.isfinite(v):
                cand[int(g)] = v
        sel, rsel = got[r][got[r] >= 0], ref[r][ref[r] >= 0]
        assert sel.size == rsel.size and np.all(got[r][sel.size:] == -1), r
        assert len(set(sel.tolist())) == sel.size and all(int(g) in cand for g in sel), r
        assert np.array_equal(np.sort([cand[int(g)] for g in sel]), np.sort([cand[int(g)] for g in rsel])), r


@pytest.mark.parametrize("R,W,k,kind", [(2, 600, 64, "plain"), (4, 5000, 512, "ties"), (8, 20000, 2048, "plain"),
                                        (3, 3000, 700, "nonfinite"), (8, 131072, 2048, "ties")])
def test_topk_merge_matches_oracle(R, W, k, kind):
    rng = np.random.default_rng(R * 1000 + k)
    rows = 6
    x, ends, vals, gidx = _candidate_lists(rng, rows, W, R, k, kind)
    ref = oracle.topk_merge(vals, gidx, k)
    got = host(dsi.topk_merge(dev(vals), dev(gidx), k=k))
    _check_merge(got, ref, vals, gidx)


def test_topk_merge_of_local_topk_is_global_topk_on_gpu():
    """The pages' exactness argument, on the device path alone: rank-local top-k over contiguous slices, their
    candidates, the merge, against the top-k of the whole rows (compared as value multisets)."""
    rng = np.random.default_rng(52)
    rows, W, R, k = 16, 65536, 8, 2048
    x = dev(rng.standard_normal((rows, W)).astype(np.float32))
    ends = dev(rng.integers(3000, W + 1, size=rows).astype(np.int32))
    full = host(dsi.topk_select(x, ends, k=k))
    L = W // R
    vals = torch.empty((R, rows, k), dtype=torch.float32, device="cuda")
    gidx = torch.empty((R, rows, k), dtype=torch.int32, device="cuda")
    for r in range(R):
        st = torch.full((rows,), r * L, dtype=torch.int32, device="cuda")
        en = torch.clamp(ends, max=(r + 1) * L)
        idx = dsi.topk_select(x, en, k=k, row_starts=st)
        dsi.topk_values(x, idx, row_starts=st, index_offset=r * L, out=(vals[r], gidx[r]))
    merged = host(dsi.topk_merge(vals, gidx, k=k))
    xh = host(x)
    for r in range(rows):
        a, b = full[r][full[r] >= 0], merged[r][merged[r] >= 0]
        assert a.size == b.size and np.array_equal(np.sort(xh[r][a]), np.sort(xh[r][b])), r


# ----------------------------------------------------------------------------- MXFP4 cache
ROW4 = 68


def _mx_pool_oracle(k_bf16, slots, nb, bs, stride, fill=0xA5):
    pool = np.full(nb * stride, fill, np.uint8)
    oracle.k_quant_and_cache_mxfp4(k_bf16, slots, pool, bs, stride)
    return pool


def test_k_quant_mxfp4_every_bf16_value_bit_exact():
    # each block of 32 holds 7.96875 (the largest bf16 below 8: shared exponent 0) and 31 sweep values, so
    # every finite bf16 value up to that size is encoded at scale 1: ties, saturation, signs, subnormals
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    vals = x[np.isfinite(x) & (np.abs(x) <= 7.96875)]
    nblk = (vals.size + 30) // 31
    flat = np.zeros(nblk * 31, np.float32)
    flat[:vals.size] = vals
    blocks = np.concatenate([np.full((nblk, 1), 7.96875, np.float32), flat.reshape(nblk, 31)], axis=1)
    n = (nblk + 3) // 4
    k = np.zeros((n * 4, 32), np.float32)
    k[:nblk] = blocks
    kb = synth._bf16_bits(k.reshape(n, 128))
    slots = np.arange(n, dtype=np.int64)
    ref = _mx_pool_oracle(kb, slots, 1, n, n * ROW4)
    pool = torch.full((n * ROW4,), 0xA5, dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache_mxfp4(dev(kb), dev(slots), pool, n, n * ROW4, 1)
    assert np.array_equal(host(pool), ref)


def test_k_quant_mxfp4_random_rows_packed_pool():
    rng = np.random.default_rng(71)
    n, bs = 1000, 64
    kb = synth.draw_k(rng, n)
    kb[0] = 0                                                                                  # zero row
    kb[1] = synth._bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(1e-38))  # subnormal-ish
    kb[2] = synth._bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(1e30))   # huge
    kb[3, 40] = synth._bf16_bits(np.array([-7.5], np.float32))[0]                               # saturating block
    stride = bs * ROW4 + 16
    nb = (n + bs - 1) // bs + 2
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[::9] = -1
    ref = _mx_pool_oracle(kb, slots, nb, bs, stride)
    pool = torch.full((nb * stride,), 0xA5, dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache_mxfp4(dev(kb), dev(slots), pool, bs, stride, nb)
    assert np.array_equal(host(pool), ref)


def test_sparse_mxfp4_exact_integer_bit_exact():
    """Keys on the FP4 grid with unit scales and q codes of small integers: every partial sum is exact, so
    the device must match the oracle bit for bit (bf16 rounding of an exact value)."""
    rng = np.random.default_rng(72)
    S, T, sbk = 512, 8, 16
    codes = rng.integers(0, 16, size=(S, 128)).astype(np.uint8)
    codes[:, ::32] = 7  # +6 in each block: shared exponent 0
    kb = synth._bf16_bits(oracle.fp4_decode(codes))
    rows4 = _mx_pool_oracle(kb, np.arange(S, dtype=np.int64), 1, S, S * ROW4)
    q = oracle.e4m3_encode(rng.integers(-8, 9, size=(T, 64, 128)).astype(np.float32))
    w = synth._bf16_bits(np.float32(2.0) ** rng.integers(-6, 0, size=(T, 64)).astype(np.float32))
    si = np.sort(rng.integers(0, S // sbk, size=(T, 12)), axis=1).astype(np.int32)
    ks, ke = np.zeros(T, np.int32), np.full(T, S, np.int32)
    end = np.full(T, 12 * sbk, np.int32)
    ref = oracle.sparse_mqa_logits_mxfp4(q, w, ks, ke, si, end, sbk, rows4)
    got = host(dsi.sparse_mqa_logits_mxfp4(dev(q), dev(w), dev(ks), dev(ke), dev(si), dev(end), sbk, dev(rows4)))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("sbk,ratio", [(128, 1), (16, 1), (8, 2)])
def test_sparse_mxfp4_gathered_parity(sbk, ratio):
    rng = np.random.default_rng(80 + sbk + ratio)
    cbs, S, T, K = sbk * ratio, 3001, 12, 16
    c = synth.prefill_case(50 + sbk, T=T, S=S, first_pos=S - T)
    rows4 = _mx_pool_oracle(c["k"], np.arange(S, dtype=np.int64), 1, S, S * ROW4)
    ks = np.zeros(T, np.int32)
    ks[3] = sbk * 2
    ke = c["ke"].copy()
    ke[5] = 40
    maxb = (np.maximum(ke - ks, 0) + cbs - 1) // cbs
    cand = synth.draw_candidates(rng, maxb, num=K, distinct=min(12, int(maxb.min())), dup=2)
    si, end = oracle.expand_candidates(cand, ks, ke, cbs, sbk)
    ref_bits = oracle.sparse_mqa_logits_mxfp4(c["q"], c["w"], ks, ke, si, end, sbk, rows4)
    ref_f32 = oracle.sparse_mqa_logits_mxfp4(c["q"], c["w"], ks, ke, si, end, sbk, rows4, out_f32=True)
    got = host(dsi.sparse_mqa_logits_mxfp4(dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(si), dev(end), sbk,
                                           dev(rows4)))
    valid = np.isfinite(ref_f32)
    assert np.array_equal(got[~valid], ref_bits[~valid])
    assert_close(bf16_value(got[valid]), ref_f32[valid], tol_fn=tol_bf16, what="MXFP4 sparse logits")


@pytest.mark.parametrize("sbk,bs", [(128, 128), (16, 64)])
def test_sparse_mxfp4_paged_parity(sbk, bs):
    rng = np.random.default_rng(sbk * 5 + bs)
    lens = [700, 1, 129, 3000, 2048]
    c = synth.decode_case(60 + sbk, B=len(lens), next_n=1, lmin=0, lmax=0, block_size=bs, lens=lens)
    stride, nb = bs * ROW4 + 16, c["num_blocks"]
    pool_np = _mx_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    rows = len(lens)
    ks = np.zeros(rows, np.int32)
    ke = np.array(lens, np.int32)
    maxb = (np.maximum(ke - ks, 0) + sbk - 1) // sbk
    cand = synth.draw_candidates(rng, maxb, num=8, distinct=6, dup=1)
    si, end = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    r2r = np.arange(rows, dtype=np.int32)
    bt = c["block_table"].copy()
    bt[3, 1] = -1  # a missing page scores -inf
    # the oracle has no missing-page rule: it scores the intact table, and the missing page's tokens are
    # masked to -inf afterwards, as the call documents
    bt_ok = c["block_table"]
    ref_f32 = oracle.sparse_mqa_logits_mxfp4(c["q"], c["w"], ks, ke, si, end, sbk, pool_np, block_table=bt_ok,
                                             row_to_req=r2r, block_size=bs, block_stride=stride, out_f32=True)
    got = host(dsi.sparse_mqa_logits_mxfp4(dev(c["q"]), dev(c["w"]), dev(ks), dev(ke), dev(si), dev(end), sbk,
                                           dev(pool_np), block_table=dev(bt), row_to_req=dev(r2r), block_size=bs,
                                           block_stride_bytes=stride, num_k=nb))
    tok = si[3][np.arange(si.shape[1] * sbk) // sbk] * sbk + np.arange(si.shape[1] * sbk) % sbk
    missing = (tok // bs) == 1
    ref_f32[3, missing] = -np.inf
    valid = np.isfinite(ref_f32)
    assert np.all(got[~valid] == 0xFF80)
    assert_close(bf16_value(got[valid]), ref_f32[valid], tol_fn=tol_bf16, what="MXFP4 sparse paged logits")


# ----------------------------------------------------------------------------- paged decode on the MXFP4 cache
@pytest.mark.parametrize("next_n,bs,extra,long", [(1, 64, 0, False), (2, 64, 16, False), (3, 16, 0, False),
                                                   (4, 32, 32, False), (1, 64, 16, True), (2, 16, 0, True)])
def test_decode_mxfp4_parity_ragged(next_n, bs, extra, long):
    """As test_decode_parity_ragged, on 68-byte MXFP4 rows (padded page strides, jobs spanning many chunks)."""
    lens = [4099, 2048 * 8 + 1, 2048 * 3 + 257, 9000] if long else [1, 15, 16, 17, 300, 1000 + next_n, 2049]
    c = synth.decode_case(80 + next_n, B=len(lens), next_n=next_n, lmin=0, lmax=0, block_size=bs, lens=lens)
    stride = bs * ROW4 + extra
    nb = c["num_blocks"]
    pool_np = _mx_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    width = max(lens) + 3
    ref = oracle.mqa_logits_paged_mxfp4(c["q"], c["w"], next_n, c["context_lens"], pool_np, bs, stride,
                                        c["block_table"], width)
    ld = width + 5
    out = torch.full((len(lens) * next_n, ld), -3.5, dtype=torch.float32, device="cuda")
    dsi.paged_mqa_logits_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_np), bs,
                                dev(c["block_table"]), width, next_n=next_n, out=out[:, :width],
                                block_stride_bytes=stride, num_blocks=nb, mxfp4=True)
    got = host(out)
    valid = np.isfinite(ref)
    assert_close(got[:, :width][valid], ref[valid], what="MXFP4 decode logits")
    assert np.all(got[:, :width][~valid] == -3.5) and np.all(got[:, width:] == -3.5)


def test_decode_mxfp4_bad_page_ids_score_minus_inf():
    c = synth.decode_case(21, B=2, next_n=1, lmin=0, lmax=0, block_size=16, lens=[64, 64])
    bs, stride, nb = 16, 16 * ROW4, c["num_blocks"]
    pool_np = _mx_pool_oracle(c["k"], c["slot_mapping"], nb, bs, stride)
    bt = c["block_table"].copy()
    bt[0, 1] = nb + 100  # out of range page
    bt[1, 2] = -7
    got = host(dsi.paged_mqa_logits_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_np), bs,
                                           dev(bt), 64, block_stride_bytes=stride, num_blocks=nb, mxfp4=True))
    assert np.all(np.isneginf(got[0, 16:32])) and np.all(np.isneginf(got[1, 32:48]))
    ref = oracle.mqa_logits_paged_mxfp4(c["q"], c["w"], 1, c["context_lens"], pool_np, bs, stride,
                                        c["block_table"], 64)
    keep = np.ones((2, 64), bool)
    keep[0, 16:32] = False
    keep[1, 32:48] = False
    assert_close(got[keep], ref[keep], what="MXFP4 decode logits")


# ----------------------------------------------------------------------------- decode logits + top-k in one call
def _fused_decode_case(seed, lens, next_n, maxc, mxfp4, bad_page_req=None):
    c = synth.decode_case(seed, B=len(lens), next_n=next_n, lmin=0, lmax=0, block_size=64, lens=lens)
    bs, nb = c["block_size"], c["num_blocks"]
    row = 68 if mxfp4 else ROW
    stride = bs * row
    quant = dsi.k_quant_and_cache_mxfp4 if mxfp4 else dsi.k_quant_and_cache
    quant_ref = oracle.k_quant_and_cache_mxfp4 if mxfp4 else oracle.k_quant_and_cache
    logits_ref = oracle.mqa_logits_paged_mxfp4 if mxfp4 else oracle.mqa_logits_paged
    pool_ref = np.zeros(nb * stride, np.uint8)
    quant_ref(c["k"], c["slot_mapping"], pool_ref, bs, stride)
    bt = c["block_table"].copy()
    if bad_page_req is not None:  # one page id out of the pool: its 64 tokens score -inf and are never selected
        bt[bad_page_req, 1] = nb + 5
    B = len(lens)
    ref = logits_ref(c["q"], c["w"], next_n, c["context_lens"], pool_ref, bs, stride,
                     np.where(bt < nb, bt, 0).astype(np.int32), maxc)
    if bad_page_req is not None:
        for i in range(next_n):
            ref[bad_page_req * next_n + i, 64:128] = -np.inf
    ends = np.minimum(np.maximum(np.repeat(c["context_lens"], next_n) - next_n + np.tile(np.arange(next_n), B) + 1, 0),
                      maxc).astype(np.int32)
    return c, pool_ref, bt, ref, ends, stride


@pytest.mark.parametrize("mxfp4", [False, True])
@pytest.mark.parametrize("next_n,lens,maxc", [
    (1, [0, 1, 100, 2047, 2048, 2049, 17000, 40000, 33333, 5000], 36000),  # split top-k, histograms in the decode kernel
    (2, [2, 100, 2049, 2050, 20000, 30000], 30000),                        # next-n rows: the top-k counts its own
])
def test_decode_topk_call_short_and_long_rows(mxfp4, next_n, lens, maxc):
    """dsi_paged_mqa_topk_decode: short rows (the -1 rule) mixed with rows long enough for the split top-k, a
    context longer than max_context_len (clipped) and a page id outside the pool; logits, selection and slot
    conversion of every row against the oracle, and the selection against the two separate calls."""
    bad = 7 if next_n == 1 else 4  # a long request
    c, pool_ref, bt, ref, ends, stride = _fused_decode_case(41 + next_n, lens, next_n, maxc, mxfp4, bad_page_req=bad)
    bs, nb, B = 64, c["num_blocks"], len(lens)
    rows = B * next_n
    pool = dev(pool_ref)
    q, w, cl, bt_t = dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(bt)
    logits = torch.full((rows, maxc + 16), 7.0, dtype=torch.float32, device="cuda")
    ws_bytes = dsi.paged_mqa_topk_decode_workspace_bytes(B, next_n, maxc)
    ws = torch.full((max(ws_bytes, 16),), 0xA5, dtype=torch.uint8, device="cuda")  # no state carried in the workspace
    _, idx_t = dsi.paged_mqa_topk_decode(q, w, cl, pool, bs, bt_t, maxc, next_n=next_n, logits=logits, workspace=ws,
                                         block_stride_bytes=stride, num_blocks=nb, mxfp4=mxfp4)
    r2r = np.repeat(np.arange(B, dtype=np.int32), next_n)
    slots = host(dsi.req_index_to_global_slot(idx_t, bt_t, bs, bs, row_to_req=dev(r2r)))
    got, idx = host(logits), host(idx_t)
    for r in range(rows):
        e = int(ends[r])
        valid = np.isfinite(ref[r])
        lost = max(0, min(e, 128) - 64) if r // next_n == bad else 0  # tokens 64..127 of the missing page
        assert valid.sum() == e - lost
        assert_close(got[r][:maxc][valid], ref[r][valid], what=f"row {r} logits")
        assert np.all(np.isneginf(got[r][:e][~valid[:e]]))
        assert np.all(got[r][e:] == 7.0), "columns past the row's range are not written"
        ref_idx = oracle.topk_select(ref[r:r + 1], ends[r:r + 1], K)[0]
        check_selection(idx[r], ref_idx, ref[r], end=e)
        n_valid = int(min(K, valid.sum()))
        assert np.all(idx[r][:n_valid] >= 0) and np.all(idx[r][n_valid:] == -1)
    exp = oracle.req_index_to_global_slot(idx, bt, bs, bs, row_to_req=r2r)
    sel_pages = np.where(idx >= 0, np.take_along_axis(np.repeat(bt, next_n, axis=0), np.maximum(idx, 0) // bs, 1), 0)
    assert np.all(sel_pages < nb), "a position on the missing page was selected"
    assert np.array_equal(slots, exp)
    # the same logits and selections as the two separate calls
    logits2 = dsi.paged_mqa_logits_decode(q, w, cl, pool, bs, bt_t, maxc, next_n=next_n, block_stride_bytes=stride,
                                          num_blocks=nb, mxfp4=mxfp4)
    idx2 = host(dsi.topk_select(logits2, dev(ends), k=K))
    g2 = host(logits2)
    for r in range(rows):
        e = int(ends[r])
        assert np.array_equal(g2[r][:e], got[r][:e])
        a, b = idx[r][idx[r] >= 0], idx2[r][idx2[r] >= 0]
        assert np.array_equal(np.sort(got[r][a]), np.sort(got[r][b]))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("k", [1, 64, 777, 2047])
def test_topk_split_smaller_k(bf16, k):
    """The split path (few long rows) with k below 2048: ordinary rows, many ties, a row with fewer than k finite
    values, and one tie value everywhere; the selected values against the oracle's."""
    rng = np.random.default_rng(71 + k + bf16)
    rows, width = 6, 60000
    x = (rng.standard_normal((rows, width)) * 30).astype(np.float32)
    x[1] = np.round(x[1] / 4) * 4
    x[2, k // 2:] = -np.inf
    x[3, :] = 0.75
    ends = np.array([width, 59999, width, 41000, 33333, width], np.int32)
    starts = np.array([0, 5, 0, 0, 1000, 17], np.int32)
    if bf16:
        bits = synth._bf16_bits(x)
        vals = bf16_value(bits)
        ref = oracle.topk_select(bits, ends, k, starts=starts, bf16=True)
        got = host(dsi.topk_select(dev(bits), dev(ends), k=k, row_starts=dev(starts)))
    else:
        vals = x
        ref = oracle.topk_select(x, ends, k, starts=starts)
        got = host(dsi.topk_select(dev(x), dev(ends), k=k, row_starts=dev(starts)))
    assert got.shape == (rows, k)
    for r in range(rows):
        check_selection(got[r], ref[r], vals[r], rule="exact", start=starts[r], end=ends[r])
        g = got[r][got[r] >= 0] + starts[r]
        o = ref[r][ref[r] >= 0] + starts[r]
        assert np.array_equal(np.sort(vals[r, g]), np.sort(vals[r, o]))
        assert np.unique(g).size == g.size
    assert np.sum(got[2] >= 0) == k // 2


@pytest.mark.parametrize("next_n,k", [(1, 300), (2, 1), (4, 2048)])
def test_decode_topk_call_other_k_and_next_n(next_n, k):
    """dsi_paged_mqa_topk_decode with k below 2048 (histograms counted in the decode kernel for one row per
    request) and with four rows per request (the plain top-k after the logits); selections against the oracle."""
    lens, maxc = [30000, 20000, 1000, 2], 30000
    c, pool_ref, bt, ref, ends, stride = _fused_decode_case(81 + next_n, lens, next_n, maxc, False)
    bs, nb = 64, c["num_blocks"]
    logits, idx_t = dsi.paged_mqa_topk_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_ref), bs,
                                              dev(bt), maxc, next_n=next_n, k=k, block_stride_bytes=stride,
                                              num_blocks=nb)
    got, idx = host(logits), host(idx_t)
    assert idx.shape == (len(lens) * next_n, k)
    for r in range(len(lens) * next_n):
        e = int(ends[r])
        assert_close(got[r][:e], ref[r][:e], what=f"row {r} logits")
        ref_idx = oracle.topk_select(ref[r:r + 1], ends[r:r + 1], k)[0]
        check_selection(idx[r], ref_idx, ref[r], end=e)
        sel = idx[r][idx[r] >= 0]
        assert sel.size == min(k, e) and np.unique(sel).size == sel.size


def test_decode_topk_call_many_requests():
    """More requests than the persistent decode grid takes (1100 > 1024): the per-request grid, and with 1100 rows
    the top-k's one-workgroup-per-row path for long rows; short rows padded with -1, one long row, a request of
    length 0.  Logits and selections of every row against the oracle."""
    rng = np.random.default_rng(97)
    B, maxc = 1100, 20000
    lens = rng.integers(1, 600, B).astype(np.int32)
    lens[5], lens[700], lens[1099] = 20000, 0, 2049
    c, pool_ref, bt, ref, ends, stride = _fused_decode_case(97, list(lens), 1, maxc, False)
    bs, nb = 64, c["num_blocks"]
    logits, idx_t = dsi.paged_mqa_topk_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), dev(pool_ref), bs,
                                              dev(bt), maxc, block_stride_bytes=stride, num_blocks=nb)
    got, idx = host(logits), host(idx_t)
    ref_idx = oracle.topk_select(ref, ends, K)
    for r in range(B):
        e = int(ends[r])
        assert_close(got[r][:e], ref[r][:e], what=f"row {r} logits")
        check_selection(idx[r], ref_idx[r], ref[r], end=e)
        assert np.sum(idx[r] >= 0) == min(K, e)
    assert np.all(idx[700] == -1)


@pytest.mark.parametrize("next_n", [1, 2])
def test_decode_topk_call_ties_and_heavy_boundary(next_n):
    """Every key of a long row equal (one logit value over 40000 columns): the boundary bin holds more columns
    than the candidate list, so the split top-k resolves it by passes over the row (its histograms counted in the
    decode kernel with one row per request, by the top-k itself with two); any 2048 of the tied columns are
    correct."""
    lens = [40000, 30000, 3000]
    c = synth.decode_case(44, B=3, next_n=next_n, lmin=0, lmax=0, block_size=64, lens=lens)
    k = np.tile(c["k"][:1], (c["k"].shape[0], 1))  # one k row everywhere: every logit of a row is the same
    bs, nb, stride = 64, c["num_blocks"], 64 * ROW
    pool = torch.zeros(nb * stride, dtype=torch.uint8, device="cuda")
    dsi.k_quant_and_cache(dev(k), dev(c["slot_mapping"]), pool, bs, stride, nb)
    logits, idx_t = dsi.paged_mqa_topk_decode(dev(c["q"]), dev(c["w"]), dev(c["context_lens"]), pool, bs,
                                              dev(c["block_table"]), 40000, next_n=next_n)
    idx, got = host(idx_t), host(logits)
    for r in range(len(lens) * next_n):
        L = lens[r // next_n] - next_n + r % next_n + 1  # the row's visible tokens
        sel = idx[r][idx[r] >= 0]
        assert sel.size == min(K, L) and np.unique(sel).size == sel.size and sel.max() < L
        assert np.all(got[r][sel] == got[r][0]) and np.all(got[r][:L] == got[r][0])


# ----------------------------------------------------------------------------- the per-step sparse schedule
def _schedule_case(seed, paged, mxfp4, sbk=64, bs=128):
    """Candidate blocks (duplicates, out-of-range ids, an unaligned start, an empty and a one-token row, a missing
    page) over K quantized twice (two layers of one step: same layout, different values)."""
    rng = np.random.default_rng(seed)
    row = 68 if mxfp4 else ROW
    quant_ref = oracle.k_quant_and_cache_mxfp4 if mxfp4 else oracle.k_quant_and_cache
    lens = [3000, 1, 700, 129, 5000, 0, 2048, 4100]
    R = len(lens)
    ks = np.zeros(R, np.int32)
    ks[2] = 3  # an unaligned start: columns before it score -inf
    ke = np.array(lens, np.int32)
    maxb = (np.maximum(ke - ks, 0) + sbk - 1) // sbk
    cand = synth.draw_candidates(rng, np.maximum(maxb, 1), num=12, distinct=8, dup=2)
    si, end = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    if paged:
        c = synth.decode_case(seed, B=R, next_n=1, lmin=0, lmax=0, block_size=bs, lens=lens)
        stride, nb = bs * row, c["num_blocks"]
        bt = c["block_table"].copy()
        bt[4, 1] = nb + 3  # a page id outside the pool
        pools = []
        for layer in range(2):
            k = synth.draw_k(np.random.default_rng(seed * 10 + layer), int(sum(lens)))
            pool = np.zeros(nb * stride, np.uint8)
            quant_ref(k, c["slot_mapping"], pool, bs, stride)
            pools.append(pool)
        kw = dict(block_table=bt, row_to_req=np.arange(R, dtype=np.int32), block_size=bs, block_stride=stride)
        q, w = c["q"], c["w"]
    else:
        S = 6000
        pc = synth.prefill_case(seed, T=R, S=S, first_pos=S - R)
        pools = []
        for layer in range(2):
            k = synth.draw_k(np.random.default_rng(seed * 10 + layer), S)
            pool = np.zeros(S * row, np.uint8)
            quant_ref(k, np.arange(S, dtype=np.int64), pool, S, S * row)
            pools.append(pool)
        kw = {}
        q, w = pc["q"], pc["w"]
    return q, w, ks, ke, si, end, pools, kw, sbk


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("mxfp4", [False, True])
def test_sparse_schedule_reused_over_two_layers(paged, mxfp4):
    """One schedule per step, reused by two layers (different K of the same layout): every column of each layer's
    scheduled logits equals the one-shot call's on that layer's K, bit for bit, and the oracle within tolerance."""
    q, w, ks, ke, si, end, pools, kw, sbk = _schedule_case(57 + paged + 2 * mxfp4, paged, mxfp4)
    once = dsi.sparse_mqa_logits_mxfp4 if mxfp4 else dsi.sparse_mqa_logits
    ref_fn = oracle.sparse_mqa_logits_mxfp4 if mxfp4 else oracle.sparse_mqa_logits
    args = dict(block_table=dev(kw["block_table"]), row_to_req=dev(kw["row_to_req"]), block_size=kw["block_size"],
                block_stride_bytes=kw["block_stride"]) if paged else {}
    ks_t, ke_t, si_t, end_t, q_t, w_t = dev(ks), dev(ke), dev(si), dev(end), dev(q), dev(w)
    pool0 = dev(pools[0])
    sched = dsi.sparse_schedule(ks_t, ke_t, si_t, end_t, sbk, pool0, mxfp4=mxfp4, **args)
    for layer, pool in enumerate(pools):
        p = dev(pool)
        got = host(dsi.sparse_mqa_logits_scheduled(q_t, w_t, sched, sbk, p, mxfp4=mxfp4))
        one = host(once(q_t, w_t, ks_t, ke_t, si_t, end_t, sbk, p, **args))
        assert np.array_equal(got, one), f"layer {layer}"
        okw = dict(kw)
        if paged:
            okw["block_table"] = np.where(kw["block_table"] < len(pool) // kw["block_stride"], kw["block_table"], 0)
        ref = ref_fn(q, w, ks, ke, si, end, sbk, pool, out_f32=True, **okw)
        if paged:  # the missing page's tokens (request 4, block 1) score -inf on the GPU
            tok = (si[4][:, None] * sbk + np.arange(sbk)[None, :]).reshape(-1)
            ref[4, (tok // kw["block_size"]) == 1] = -np.inf
        valid = np.isfinite(ref)
        assert np.all(got[~valid] == 0xFF80), f"layer {layer}"
        assert_close(bf16_value(got[valid]), ref[valid], tol_fn=tol_bf16, what=f"layer {layer} scheduled logits")


@pytest.mark.parametrize("mxfp4", [False, True])
@pytest.mark.parametrize("sbk", [8, 16, 128])
def test_sparse_schedule_long_rows_small_blocks(sbk, mxfp4):
    """Rows of 10240 candidate columns (40 chunks of 256) in blocks of 8, 16 and 128 tokens: the scheduled call
    spans several segments per row (the FP8 kernel's segment is min(32, sbk) chunks, so at 8 tokens per block
    its 256 staged entries are full) and segments that start inside a row; every column equals the one-shot
    call's, bit for bit."""
    rng = np.random.default_rng(71 + sbk + mxfp4)
    R, S, width = 6, 12000, 10240
    row = 68 if mxfp4 else ROW
    quant_ref = oracle.k_quant_and_cache_mxfp4 if mxfp4 else oracle.k_quant_and_cache
    once = dsi.sparse_mqa_logits_mxfp4 if mxfp4 else dsi.sparse_mqa_logits
    pc = synth.prefill_case(80 + sbk, T=R, S=S, first_pos=S - R)
    ks = np.zeros(R, np.int32)
    ks[1] = 5 * sbk + 3  # an unaligned start
    ke = (S - R + 1 + np.arange(R)).astype(np.int32)
    maxb = (np.maximum(ke - ks, 0) + sbk - 1) // sbk
    num = width // sbk
    cand = synth.draw_candidates(rng, maxb, num=num, distinct=num - 4, dup=2)
    # (the oracle's expansion: 1280 sparse blocks per row at 8 tokens exceed the expansion kernel's 1024)
    si_np, end_np = oracle.expand_candidates(cand, ks, ke, sbk, sbk)
    si, end = dev(si_np), dev(end_np)
    k = synth.draw_k(np.random.default_rng(90 + sbk), S)
    pool = np.zeros(S * row, np.uint8)
    quant_ref(k, np.arange(S, dtype=np.int64), pool, S, S * row)
    p, q_t, w_t, ks_t, ke_t = dev(pool), dev(pc["q"]), dev(pc["w"]), dev(ks), dev(ke)
    sched = dsi.sparse_schedule(ks_t, ke_t, si, end, sbk, p, mxfp4=mxfp4)
    got = host(dsi.sparse_mqa_logits_scheduled(q_t, w_t, sched, sbk, p, mxfp4=mxfp4))
    one = host(once(q_t, w_t, ks_t, ke_t, si, end, sbk, p))
    assert got.shape == (R, width)
    assert np.array_equal(got, one)
    assert (got != np.int16(-128)).sum() > R * width // 2  # most columns score (0xFF80 is -inf)


def test_sparse_schedule_bounds_the_source():
    """A schedule built for a larger source than the one scored: columns whose rows lie past the given source's
    size score -inf instead of reading outside it."""
    q, w, ks, ke, si, end, pools, kw, sbk = _schedule_case(61, False, False)
    sched = dsi.sparse_schedule(dev(ks), dev(ke), dev(si), dev(end), sbk, dev(pools[0]))
    half = dev(pools[0][: (len(pools[0]) // 2 // ROW) * ROW])  # the first 3000 rows only
    got = host(dsi.sparse_mqa_logits_scheduled(dev(q), dev(w), sched, sbk, half))
    full = host(dsi.sparse_mqa_logits_scheduled(dev(q), dev(w), sched, sbk, dev(pools[0])))
    tok = (si[:, :, None] * sbk + np.arange(sbk)[None, None, :]).reshape(si.shape[0], -1)
    inside = tok < 3000
    assert np.array_equal(got[inside], full[inside])
    assert np.all(got[~inside] == 0xFF80)


@pytest.mark.parametrize("width", [4096, 8192, 16384, 40000])
def test_topk_extreme_values_and_non_finite(width):
    """Boundaries at both ends of the finite range: values next to the largest float (the
    top first-digit bin), next to minus the largest, and rows mixing them with +-inf and +-NaN
    (never selected), in fp32 and bf16, for each row-length path."""
    rng = np.random.default_rng(width)
    fmax = np.finfo(np.float32).max
    near_top = lambda n: (fmax * (1 - rng.uniform(0, 2 ** -10, n))).astype(np.float32)
    rows = 6
    x = rng.standard_normal((rows, width)).astype(np.float32)
    x[0, :3000] = near_top(3000)                        # boundary in the top bin
    x[1, :] = -fmax                                     # all equal, lowest finite bin
    x[1, :2] = [np.inf, np.nan]
    x[2, ::4] = np.inf
    x[2, 1::4] = np.nan
    x[2, 2::4] = -np.inf
    x[2, 3::8] = near_top(len(x[2, 3::8]))
    x[3] = rng.permutation(np.concatenate([near_top(width // 2), -near_top(width - width // 2)]))
    x[4, :] = np.float32(-np.nan)                       # negative NaN everywhere: nothing valid
    x[4, :5] = 1.0
    x[5, : width // 2] = np.inf
    for r in range(rows):
        x[r] = rng.permutation(x[r])
    ends = np.full(rows, width, np.int32)
    ref = oracle.topk_select(x, ends, 2048)
    got = host(dsi.topk_select(dev(x), dev(ends), k=2048))
    for r in range(rows):
        check_selection(got[r], ref[r], x[r], rule="exact", end=width)
    if width > 16384:
        return
    bits = synth._bf16_bits(rng.standard_normal((rows, width)).astype(np.float32))
    bits[0, :3000] = 0x7F7F - rng.integers(0, 2, 3000).astype(np.uint16)  # the two largest bf16 values
    bits[1, :] = 0xFF7F                                                  # minus the largest, everywhere
    bits[2, ::4] = 0x7F80
    bits[2, 1::4] = 0x7FC0
    bits[2, 2::4] = 0xFF80
    bits[3, 3::2] = 0xFFC0                                               # negative NaN
    bits[4, :] = 0xFFC1
    bits[5, : width // 2] = 0x7F80
    for r in range(rows):
        bits[r] = rng.permutation(bits[r])
    ref = oracle.topk_select(bits, ends, 2048, bf16=True)
    got = host(dsi.topk_select(dev(bits), dev(ends), k=2048))
    f = bf16_value(bits)
    for r in range(rows):
        check_selection(got[r], ref[r], f[r], rule="exact", end=width)
