"""Pins for the oracle's q preparation (RoPE on the first 64 dims, FP8 quantization, weight fold).

Page "DeepSeek V3.2 sparse attention DSA inference flow", indexer steps ③ (RoPE on the first 64 of 128 dims only)
and ④ (one FP8 scale per 128 values of q; weights * q_scale * softmax_scale * head_scale), pitfalls (the indexer's
RoPE has its own interleave switch).  Page "V4.1 indexer uses sparse MQA logits", implementation breakdown: the
fused q kernel writes bf16 weights equal to the fp32 result rounded once.

Pins: angles whose cosine and sine are exactly 0 or +-1 reduce the rotation to a permutation with sign changes,
so the codes must equal the (separately pinned) k quantization of the hand-permuted vector; random angles are
checked against an fp64 rotation within the E4M3 error bound; the weights against the library's bf16 rounding
of the fp32 product and against fp64.
"""
import numpy as np
import torch

import oracle
import synth

H, D = 64, 128


def _kquant(x_bits):
    """k quantization oracle on rows [n,128] of bf16 bits -> (codes [n,128], scales [n])."""
    n = x_bits.shape[0]
    pool = np.zeros(n * 132, dtype=np.uint8)
    oracle.k_quant_and_cache(x_bits, np.arange(n, dtype=np.int64), pool, n, n * 132)
    rows = pool.reshape(n, 132)
    return rows[:, :128].copy(), rows[:, 128:].copy().view(np.float32)[:, 0]


def _table(cos, sin):
    return np.concatenate([np.full(32, cos, np.float32), np.full(32, sin, np.float32)])[None, :]


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).bfloat16().view(torch.int16).numpy().view(np.uint16)


def test_zero_angle_is_plain_quantization_and_fold():
    c = synth.q_prep_case(21, 6)
    pos = np.zeros(6, np.int64)
    q8, w = oracle.q_rope_quant(c["q"], pos, _table(1.0, 0.0), c["w"], c["softmax_scale"], c["head_scale"])
    codes, scales = _kquant(c["q"].reshape(-1, D))
    assert np.array_equal(q8.reshape(-1, D), codes)
    wf = synth._bf16_value(c["w"]).reshape(-1)
    prod = ((wf * scales) * np.float32(c["softmax_scale"])) * np.float32(c["head_scale"])  # fp32, in order
    assert prod.dtype == np.float32
    assert np.array_equal(w.reshape(-1), _bf16(prod))
    exact = wf.astype(np.float64) * scales * c["softmax_scale"] * c["head_scale"]
    assert np.all(np.abs(synth._bf16_value(w.reshape(-1)) - exact) <= 2.0 ** -8 * np.abs(exact) * 1.0001)


def _rot_expect(x, cos, sin, interleave):
    """The rotation by an angle with cos, sin in {0, +-1}, as an index permutation with signs."""
    y = x.copy()
    for i in range(32):
        a, b = (2 * i, 2 * i + 1) if interleave else (i, i + 32)
        y[..., a] = x[..., a] * cos - x[..., b] * sin
        y[..., b] = x[..., b] * cos + x[..., a] * sin
    return y


def test_quarter_and_half_turns_permute_exactly():
    c = synth.q_prep_case(22, 4)
    xf = synth._bf16_value(c["q"])
    for interleave in (False, True):
        for cos, sin in ((0.0, 1.0), (-1.0, 0.0), (0.0, -1.0)):
            q8, _ = oracle.q_rope_quant(c["q"], np.zeros(4, np.int64), _table(cos, sin), c["w"], 1.0, 1.0,
                                        interleave=interleave)
            y = _rot_expect(xf, cos, sin, interleave)
            # the permuted values are bf16 values again (exact), so the k oracle can quantize them
            yb = synth._bf16_bits(y)
            assert np.array_equal(synth._bf16_value(yb), y)
            codes, _ = _kquant(yb.reshape(-1, D))
            assert np.array_equal(q8.reshape(-1, D), codes), (interleave, cos, sin)
    # the two layouts really differ on a quarter turn
    a, _ = oracle.q_rope_quant(c["q"], np.zeros(4, np.int64), _table(0.0, 1.0), c["w"], 1.0, 1.0)
    b, _ = oracle.q_rope_quant(c["q"], np.zeros(4, np.int64), _table(0.0, 1.0), c["w"], 1.0, 1.0, interleave=True)
    assert not np.array_equal(a, b)


def test_random_angles_within_e4m3_bound_of_fp64_rotation():
    c = synth.q_prep_case(23, 16, max_pos=4096)
    cs = c["cos_sin"].astype(np.float64)
    x = synth._bf16_value(c["q"]).astype(np.float64)
    for interleave in (False, True):
        q8, _ = oracle.q_rope_quant(c["q"], c["positions"], c["cos_sin"], c["w"], 1.0, 1.0, interleave=interleave)
        y = x.copy()
        for t, p in enumerate(c["positions"]):
            for i in range(32):
                a, b = (2 * i, 2 * i + 1) if interleave else (i, i + 32)
                co, si = cs[p, i], cs[p, 32 + i]
                y[t, :, a] = x[t, :, a] * co - x[t, :, b] * si
                y[t, :, b] = x[t, :, b] * co + x[t, :, a] * si
        scale = np.maximum(np.abs(y).max(axis=-1, keepdims=True), 1e-4) / 448.0
        dec = oracle.e4m3_decode(q8).astype(np.float64) * scale
        err = np.abs(dec - y)
        # E4M3: half an ulp = 2^-4 relative for normal codes, 2^-10 * scale absolute at the subnormal end,
        # plus the fp32 rotation's own rounding
        assert np.all(err <= 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * scale + 1e-6 * scale * 448), interleave


def test_positions_outside_the_table_give_zero_rows():
    c = synth.q_prep_case(24, 3, max_pos=8)
    pos = np.array([-1, 8, 3], np.int64)
    q8, w = oracle.q_rope_quant(c["q"], pos, c["cos_sin"], c["w"], c["softmax_scale"], c["head_scale"])
    assert not q8[:2].any() and not w[:2].any() and q8[2].any() and w[2].any()
