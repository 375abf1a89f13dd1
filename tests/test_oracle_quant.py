"""Pins for the oracle's k quantization fused with cache insertion.

Page "DeepSeek V3.2 sparse attention DSA inference flow": indexer step ⑤ (k quantized and written to the
cache in one operation) and the 132-byte cache row of the data-flow section (128 FP8 codes + fp32 scale).
"""
import numpy as np
import torch

import oracle
import synth


def _pool(nblocks, stride, fill=0xA5):
    return np.full(nblocks * stride, fill, dtype=np.uint8)


def _row(pool, slot, bs, stride):
    a = (slot // bs) * stride + (slot % bs) * 132
    return pool[a:a + 128], pool[a + 128:a + 132].view(np.float32)[0]


def test_zero_row():
    k = np.zeros((1, 128), dtype=np.uint16)
    pool = _pool(1, 64 * 132)
    oracle.k_quant_and_cache(k, np.array([5]), pool, 64, 64 * 132)
    codes, scale = _row(pool, 5, 64, 64 * 132)
    assert np.all(codes == 0)
    assert scale == np.float32(1e-4) / np.float32(448.0)


def test_exact_grid_row_reproduces_codes():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=128).astype(np.uint8)
    codes[(codes & 0x7F) >= 0x7E] = 0x30  # keep |code| below max ...
    codes[17] = 0x7E  # ... except one element at +448 that sets amax
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * np.float32(0.125)  # amax = 56
    k = synth._bf16_bits(vals)[None, :]
    assert np.array_equal(synth._bf16_value(k[0]), vals)  # exactly representable in bf16
    pool = _pool(1, 4 * 132)
    oracle.k_quant_and_cache(k, np.array([2]), pool, 4, 4 * 132)
    got, scale = _row(pool, 2, 4, 4 * 132)
    assert scale == np.float32(0.125)
    # +0 and -0 both decode to zero; compare codes with the sign of zero normalised
    z = (codes & 0x7F) == 0
    assert np.array_equal(got[~z], codes[~z]) and np.all((got[z] & 0x7F) == 0)


def test_error_bound_random_rows():
    rng = np.random.default_rng(3)
    k = synth.draw_k(rng, 500)
    pool = _pool(8, 64 * 132)
    oracle.k_quant_and_cache(k, np.arange(500), pool, 64, 64 * 132)
    x = synth._bf16_value(k)
    for i in range(500):
        codes, scale = _row(pool, i, 64, 64 * 132)
        amax = np.abs(x[i]).max()
        assert scale == np.float32(max(amax, np.float32(1e-4))) / np.float32(448.0)
        dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        err = np.abs(dec * scale - x[i])
        # half an ulp of a 3-bit mantissa (2^-4 relative), or half the subnormal step 2^-10 * scale
        bound = np.maximum(2.0 ** -4 * np.abs(x[i]), 2.0 ** -10 * scale) * (1 + 1e-6)
        assert np.all(err <= bound)
        assert codes[np.argmax(np.abs(x[i]))] & 0x7F == 0x7E  # the amax element hits +-448


def test_slots_layout_skip_and_packed_stride():
    rng = np.random.default_rng(4)
    k = synth.draw_k(rng, 6)
    bs, stride = 4, 4 * 132 + 16  # packed: 16 spare bytes per block
    pool = _pool(3, stride)
    slots = np.array([6, -1, 0, 11, 3, -1], dtype=np.int64)
    oracle.k_quant_and_cache(k, slots, pool, bs, stride)
    ref = _pool(3, stride)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        one = _pool(1, 132)
        oracle.k_quant_and_cache(k[i:i + 1], np.array([0]), one, 1, 132)
        a = (s // bs) * stride + (s % bs) * 132
        ref[a:a + 132] = one
    assert np.array_equal(pool, ref)
    # the 16 spare bytes of every block and the rows of unused slots stay untouched
    for b in range(3):
        assert np.all(pool[b * stride + 4 * 132:(b + 1) * stride] == 0xA5)


def test_codes_match_library_cast():
    rng = np.random.default_rng(5)
    k = synth.draw_k(rng, 200)
    pool = _pool(4, 64 * 132)
    oracle.k_quant_and_cache(k, np.arange(200), pool, 64, 64 * 132)
    x = torch.from_numpy(synth._bf16_value(k))
    scale = torch.clamp(x.abs().amax(-1, keepdim=True), min=1e-4) / 448.0
    ref = torch.clamp(x / scale, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i in range(200):
        codes, _ = _row(pool, i, 64, 64 * 132)
        assert np.array_equal(codes, ref[i])
