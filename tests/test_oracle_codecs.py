"""Pins for the oracle's FP8 (OCP e4m3fn) and bf16 codecs against library routines and closed values.

The indexer stores FP8 q and k ("DeepSeek V3.2 sparse attention DSA inference flow", cost table and
indexer step ④); the hierarchical path writes bf16 logits (vLLM PR 56254 summary, implementation).
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def torch_e4m3_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])


def test_decode_hand_values():
    d = oracle.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0xB8, 0x00, 0x80], dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -9 and d[3] == 2.0 ** -6
    assert d[4] == 7 * 2.0 ** -9 and d[5] == -1.0 and d[6] == 0.0 and d[7] == 0.0 and np.signbit(d[7])


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_encode_all_bf16_in_range_matches_torch():
    # every bf16 bit pattern with |x| < 448: covers every e4m3 midpoint (ties) and the subnormal range
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 448)]
    assert np.array_equal(oracle.e4m3_encode(x), torch_e4m3_encode(x))


def test_encode_random_fp32_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-447.9, 447.9, 20000), rng.standard_normal(20000) * 0.01]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), torch_e4m3_encode(x))


def test_encode_ties_go_to_even_mantissa():
    # 1 + 1/16 lies halfway between 1 (m=0) and 1.125 (m=1): even -> 1.0
    # 1 + 3/16 lies halfway between 1.125 (m=1) and 1.25 (m=2): even -> 1.25
    # 3 * 2^-10 lies halfway between 1*2^-9 (m=1) and 2*2^-9 (m=2): even -> code 2
    e = oracle.e4m3_encode(np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10], dtype=np.float32))
    assert list(e) == [0x38, 0x3A, 0x02, 0x00]


def test_encode_saturates():
    e = oracle.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, -500.0, -1e30], dtype=np.float32))
    assert list(e) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_encode_keeps_sign_of_zero():
    e = oracle.e4m3_encode(np.array([0.0, -0.0, -1e-9, 1e-9], dtype=np.float32))
    assert list(e) == [0x00, 0x80, 0x80, 0x00]


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * 100, rng.standard_normal(1000) * 1e-30,
                        rng.standard_normal(1000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(x), ref)


def test_bf16_hand_values():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.0, float("inf"), float("-inf")], dtype=np.float32)
    assert list(oracle.bf16_rne(x)) == [0x3F80, 0x3F82, 0xC000, 0x7F80, 0xFF80]
    assert oracle.bf16_to_f32(np.array([0x3F82], dtype=np.uint16))[0] == 1 + 2.0 ** -6
