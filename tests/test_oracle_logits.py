"""Pins for the oracle's indexer logits.

Definition ("DeepSeek V3.2 sparse attention DSA inference flow", indexer step ⑥): the score of history
token s for query token t is the weighted sum over the 64 heads of the head's dot product with the one
shared 128-d key, logits[t,s] = sum_h w[t,h] (q[t,h] . k[s]).  Prefill scores gathered K, decode reads the
paged cache directly (same page, prefill/decode table).
"""
import numpy as np
import torch

import oracle
import synth

U = 2.0 ** -24


def dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def kvals(k_rows):
    scale = np.ascontiguousarray(k_rows[:, 128:132]).view(np.float32)[:, 0].astype(np.float64)
    return dec(k_rows[:, :128]), scale


def small_case(seed, T=5, S=70):
    c = synth.prefill_case(seed, T=T, S=S, first_pos=S - T)
    rows = np.zeros((S, 132), dtype=np.uint8)
    flat = rows.reshape(-1)
    oracle.k_quant_and_cache(c["k"], np.arange(S), flat, S, S * 132)
    return c, rows


def exact_and_bound(q, w, k_rows):
    """fp64 brute force of the definition, and the fp32 rounding bound of the oracle's evaluation."""
    qv = dec(q)  # [T,64,128]
    wv = synth._bf16_value(w).astype(np.float64)  # [T,64]
    kc, ks = kvals(k_rows)
    kd = kc * ks[:, None]  # [S,128]
    terms = np.einsum("thd,sd->tsh", qv, kd)  # per-head dots
    exact = np.einsum("th,tsh->ts", wv, terms)
    absum = np.einsum("th,thd,sd->ts", np.abs(wv), np.abs(qv), np.abs(kd))
    return exact, absum * 260 * U


def test_definition_fp64_brute_force():
    c, rows = small_case(11)
    got = oracle.mqa_logits_gathered(c["q"], c["w"], rows, c["ks"], c["ke"])
    exact, bound = exact_and_bound(c["q"], c["w"], rows)
    valid = np.arange(c["S"])[None, :] < c["ke"][:, None]
    assert np.all(np.abs(got[valid] - exact[valid]) <= bound[valid])
    assert np.all(np.isneginf(got[~valid]))


def test_head_collapse_identity_fp64():
    # sum_h w_h (q_h . k) == (sum_h w_h q_h) . k, evaluated in fp64 by a different route
    c, rows = small_case(12)
    got = oracle.mqa_logits_gathered(c["q"], c["w"], rows, c["ks"], c["ke"])
    qv, wv = dec(c["q"]), synth._bf16_value(c["w"]).astype(np.float64)
    kc, ks = kvals(rows)
    v = np.einsum("th,thd->td", wv, qv)
    ref = (v @ (kc * ks[:, None]).T)
    _, bound = exact_and_bound(c["q"], c["w"], rows)
    valid = np.arange(c["S"])[None, :] < c["ke"][:, None]
    assert np.all(np.abs(got[valid] - ref[valid]) <= bound[valid] + 1e-9 * np.abs(ref[valid]))


def int_code(v):
    """e4m3 code of a small integer -8..8 (exact)."""
    table = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E, 8: 0x50}
    c = table[abs(int(v))]
    return c | (0x80 if v < 0 else 0)


def exact_int_case(rng, T, S):
    qi = rng.integers(-8, 9, size=(T, 64, 128))
    ki = rng.integers(-8, 9, size=(S, 128))
    e = rng.integers(-3, 4, size=(T, 64))
    sgn = rng.choice([-1.0, 1.0], size=(T, 64))
    wf = (sgn * 2.0 ** e).astype(np.float32)
    q = np.vectorize(int_code)(qi).astype(np.uint8)
    rows = np.zeros((S, 132), dtype=np.uint8)
    rows[:, :128] = np.vectorize(int_code)(ki).astype(np.uint8)
    rows[:, 128:132] = np.ones(S, dtype=np.float32).view(np.uint8).reshape(S, 4)
    w = synth._bf16_bits(wf)
    # exact integer arithmetic (int64 with the power-of-two weights as rationals over 8)
    w8 = (wf * 8).astype(np.int64)
    ref8 = np.einsum("th,thd,sd->ts", w8, qi, ki)
    return q, w, rows, ref8 / 8.0


def test_exact_integer_case_bit_exact():
    rng = np.random.default_rng(13)
    q, w, rows, ref = exact_int_case(rng, 3, 40)
    got = oracle.mqa_logits_gathered(q, w, rows, np.zeros(3, np.int32), np.full(3, 40, np.int32))
    assert np.array_equal(got.astype(np.float64), ref)


def test_linearity_in_weights_power_of_two():
    c, rows = small_case(14, T=3, S=50)
    a = oracle.mqa_logits_gathered(c["q"], c["w"], rows, c["ks"], c["ke"])
    w2 = synth._bf16_bits(synth._bf16_value(c["w"]) * np.float32(4.0))
    b = oracle.mqa_logits_gathered(c["q"], w2, rows, c["ks"], c["ke"])
    valid = np.isfinite(a)
    assert np.array_equal(b[valid], a[valid] * np.float32(4.0))


def test_paged_addressing_equals_gathered():
    # build a paged pool from gathered rows with numpy indexing under a permuted block table
    rng = np.random.default_rng(15)
    bs, L = 16, 75
    c, rows = small_case(16, T=2, S=L)
    nblk = (L + bs - 1) // bs
    perm = rng.permutation(nblk + 3).astype(np.int32)[:nblk]
    stride = bs * 132 + 32  # packed block stride
    pool = np.zeros((nblk + 3) * stride, dtype=np.uint8)
    for s in range(L):
        a = perm[s // bs] * stride + (s % bs) * 132
        pool[a:a + 132] = rows[s]
    # request of length L with next_n = 2: rows see [0, L-1) and [0, L)
    paged = oracle.mqa_logits_paged(c["q"], c["w"], 2, np.array([L], np.int32), pool, bs, stride, perm[None, :],
                                    width=L + 5)
    gathered = oracle.mqa_logits_gathered(c["q"], c["w"], rows, np.zeros(2, np.int32),
                                          np.array([L - 1, L], np.int32))
    assert np.array_equal(paged[:, :L], gathered)
    assert np.all(np.isneginf(paged[:, L:]))
    assert np.isneginf(paged[0, L - 1]) and np.isfinite(paged[1, L - 1])


def test_row_ranges_mask():
    c, rows = small_case(17, T=4, S=30)
    ks = np.array([0, 5, 10, 29], np.int32)
    ke = np.array([30, 6, 10, 30], np.int32)
    got = oracle.mqa_logits_gathered(c["q"], c["w"], rows, ks, ke)
    s = np.arange(30)
    assert np.array_equal(np.isfinite(got), (s[None, :] >= ks[:, None]) & (s[None, :] < ke[:, None]))
