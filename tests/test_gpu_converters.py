"""The device converters the kernels rely on, over their whole input ranges, against the CPU oracle (the codecs
are pinned to the format definitions by tests/test_oracle_codecs.py and tests/test_oracle_mxfp4.py):

  * fp32 -> E4M3FN on the hardware encoder (q preparation) for every fp32 bit pattern with |x| <= 464, both signs.
    The probe reports where the code changes; the oracle is checked at both ends of every run of equal codes.
    Round-to-nearest is monotone in |x| (pinned by the oracle's codec tests), so equal codes at both ends of a
    run mean equal codes on all of it: the comparison covers all 2.27e9 patterns.
  * E4M3FN -> f16 and -> bf16 for all 256 codes (every logits kernel's operand decode; the MXFP4 kernels' q).
  * FP4 E2M1 x E8M0 scale -> bf16 for all 16 codes and all 256 scale bytes (the MXFP4 key decode): exact for
    scales up to 2^125 (E <= 252); larger ones overflow, as they do in fp32.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_token_amd import probe

pytestmark = pytest.mark.gpu

F464 = 0x43E80000  # the bit pattern of 464.0


def _f32(u):
    return float(np.array([u], dtype=np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_hw_e4m3_encoder_on_every_fp32_up_to_464(sign):
    first, changes = probe.e4m3_encode_changes(sign, F464 + 1)
    # runs of equal codes: [start, next start - 1]
    starts = [sign] + [u for u, _ in changes]
    codes = [first] + [c for _, c in changes]
    ends = [u - 1 for u, _ in changes] + [sign + F464]
    assert len(changes) <= 130  # one change per code boundary (126 per sign), no jitter
    for lo, hi, c in zip(starts, ends, codes):
        assert lo <= hi
        assert int(oracle.e4m3_encode(np.float32(_f32(lo)))) == c, (hex(lo), c)
        assert int(oracle.e4m3_encode(np.float32(_f32(hi)))) == c, (hex(hi), c)
    assert codes[-1] == (0xFE if sign else 0x7E)  # saturation at 448


def test_hw_e4m3_decode_to_f16_and_bf16_all_codes():
    f16, bf16 = probe.e4m3_decode_all()
    ref = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(nan, (np.arange(256) & 0x7F) == 0x7F)
    got16 = f16.view(np.float16).astype(np.float32)
    assert np.all(np.isnan(got16[nan]))
    assert np.array_equal(got16[~nan], ref[~nan])  # every finite E4M3 value is a normal f16: exact
    assert np.array_equal(np.signbit(got16[~nan]), np.signbit(ref[~nan]))  # -0 stays -0
    gotb = (bf16.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(gotb[nan]))
    assert np.array_equal(gotb[~nan], ref[~nan])
    assert np.array_equal(np.signbit(gotb[~nan]), np.signbit(ref[~nan]))


def test_hw_fp4_decode_all_codes_and_scales():
    got = probe.fp4_decode_all()  # [256 scale bytes][16 codes]
    vals = oracle.fp4_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    for e in range(253):
        ref = vals * 2.0 ** (e - 127)  # exact in float64, and a bf16 value for every code at these scales
        ref32 = ref.astype(np.float32)
        assert np.array_equal(ref32.astype(np.float64), ref)
        g = (got[e].astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(g, ref32), e
        assert np.array_equal(np.signbit(g), np.signbit(ref32)), e
