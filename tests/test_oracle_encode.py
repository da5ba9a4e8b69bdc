"""Pins of the oracle's record encoder (oracle/encode.py) against what the formats and the
mathematics fix: torch's float8_e4m3fn cast (round to nearest, ties to even), hand-derived tie and
saturation cases, the closed form of the power-of-two scale, the pages' nibble order, and the
round-trip bound dequant(encode(x)) - x <= half a step of the element grid."""
import math

import numpy as np
import pytest
import torch

from oracle import (E2M1, E4M3, dequant_fp4_records, dequant_fp8_records, e2m1_encode, e4m3_encode,
                    encode_fp4_records, encode_fp8_records, fp8_scale_exponent)


def _torch_e4m3(x):
    """torch's cast from float32 (from float64 it rounds to float32 first, a double rounding)."""
    x32 = np.asarray(x, dtype=np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def test_e4m3_matches_torch_on_values_and_every_midpoint():
    pos = E4M3[:0x7F]                                   # 0 and the finite positive values
    mids = (pos[:-1] + pos[1:]) / 2                     # exact ties
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-12, 1, 20000))
    rand = rand.astype(np.float32).astype(np.float64)
    m32 = mids.astype(np.float32)
    below = np.nextafter(m32, np.float32(0)).astype(np.float64)
    above = np.nextafter(m32, np.float32(1000)).astype(np.float64)
    for x in (pos, -pos[1:], mids, -mids, rand, below, above):
        assert np.array_equal(e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_ties_go_to_the_even_code():
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): even code 0x38; 1.1875 between 0x39 and
    # 0x3A (1.25): even 0x3A; the subnormal tie 1.5 * 2^-9 between 0x01 and 0x02 -> 0x02
    assert e4m3_encode(np.array([1.0625, 1.1875, 1.5 * 2 ** -9, 0.5 * 2 ** -9]))\
        .tolist() == [0x38, 0x3A, 0x02, 0x00]
    assert e4m3_encode(np.array([-1.0625, -0.0, -2 ** -12])).tolist() == [0xB8, 0x80, 0x80]
    # 448 is the largest finite value; beyond it the encoder saturates (only the fp4 scale can get
    # there, and only for blocks whose values exceed the fp4 format's range)
    assert e4m3_encode(np.array([448.0, 460.0, 1e6])).tolist() == [0x7E, 0x7E, 0x7E]


def test_e2m1_hand_worked_ties_and_saturation():
    x = np.array([0.0, 0.25, 0.26, 0.74, 0.75, 1.25, 1.26, 1.75, 2.5, 2.6, 3.5, 5.0, 5.1, 6.0, 7.0, 1e9])
    assert e2m1_encode(x).tolist() == [0, 0, 1, 1, 2, 2, 3, 4, 4, 5, 6, 6, 7, 7, 7, 7]
    assert e2m1_encode(-x).tolist() == [c | 8 for c in [0, 0, 1, 1, 2, 2, 3, 4, 4, 5, 6, 6, 7, 7, 7, 7]]
    # every code is the encoding of its own value (-0 encodes as code 8)
    for c in range(16):
        v = -0.0 if c == 8 else E2M1[c]
        assert e2m1_encode(np.array([v]))[0] == c


def test_fp8_scale_exponent_closed_form():
    # amax = M * 2^E with M in [1, 2): k = E - 8 when M <= 1.75, E - 7 above (448 = 1.75 * 2^8)
    rng = np.random.default_rng(1)
    amax = _bf16(np.abs(rng.standard_normal(5000)) * np.exp2(rng.integers(-60, 60, 5000)))
    amax = amax[amax > 0]
    m, e = np.frexp(amax)                               # amax = m * 2^e, m in [0.5, 1)
    expect = (e - 1) - 8 + (2 * m > 1.75)
    assert np.array_equal(fp8_scale_exponent(amax), np.clip(expect, -127, 127))
    assert fp8_scale_exponent(np.array([448.0, 449.0, 224.0, 1.0, 0.0, 7 * 2.0 ** 100])).tolist() \
        == [0, 1, -1, -8, 0, 94]
    assert fp8_scale_exponent(np.array([2.0 ** -133, 3e38])).tolist() == [-127, 120]


def test_fp8_record_layout_and_round_trip():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-20, 20, (64, 16, 1)))
              .repeat(32, axis=2).reshape(64, 512))
    rec = encode_fp8_records(x)
    assert rec.shape == (64, 528)
    blocks = x.reshape(64, 16, 32)
    k = fp8_scale_exponent(np.abs(blocks).max(axis=2))
    assert np.array_equal(rec[:, 512:], (k + 127).astype(np.uint8))        # scale j after the data
    y = blocks / np.exp2(k)[:, :, None]
    assert np.abs(y).max() <= 448
    assert np.array_equal(rec[:, :512], _torch_e4m3(y.reshape(64, 512)))
    # round trip: within half a step of the e4m3 grid at each value's magnitude
    back = dequant_fp8_records(rec).reshape(64, 16, 32)
    mag = np.abs(y)
    step = np.where(mag >= 2 ** -6, np.exp2(np.floor(np.log2(np.maximum(mag, 2 ** -6))) - 3), 2 ** -9)
    assert np.all(np.abs(back - blocks) <= step / 2 * np.exp2(k)[:, :, None])


def test_fp8_all_zero_block_and_block_at_the_limit():
    x = np.zeros((1, 512))
    x[0, 32] = 448.0                                     # block 1 exactly at the e4m3 limit
    x[0, 64] = -449.0                                    # block 2 just above: scale 2^1
    rec = encode_fp8_records(x)
    assert rec[0, 512] == 127 and rec[0, 513] == 127 and rec[0, 514] == 128
    assert rec[0, 32] == 0x7E and rec[0, 64] == 0xF6    # -449 / 2 = -224.5 -> -224 (0xF6)
    assert np.all(rec[0, :32] == 0)


def test_fp4_record_layout_nibble_order_and_scales():
    x = np.zeros((1, 512))
    x[0, 0], x[0, 1], x[0, 15] = 0.5, 1.0, 6.0           # block 0: amax 6 -> scale 1.0 (0x38)
    x[0, 16:32] = -3.0                                   # block 1: amax 3 -> scale 0.5 (0x30)
    rec = encode_fp4_records(x)
    assert rec.shape == (1, 288)
    assert rec[0, 0] == 0x21                             # even index in the low nibble
    assert rec[0, 7] == 0x70                             # x[14] = 0 (low), x[15] = 6 (code 7, high)
    assert rec[0, 256] == 0x38 and rec[0, 257] == 0x30
    assert np.all(rec[0, 8:16] == 0xFF)                  # -3 / 0.5 = -6 -> code 15, both nibbles
    assert np.all(rec[0, 258:] == 0x38)                  # all-zero blocks store the scale 1.0
    assert np.array_equal(dequant_fp4_records(rec)[0], x[0])


def test_fp4_scale_is_the_nearest_e4m3_of_amax_over_6_and_round_trip():
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-6, 6, (64, 32, 1)))
              .repeat(16, axis=2).reshape(64, 512))
    rec = encode_fp4_records(x)
    amax = np.abs(x.reshape(64, 32, 16)).max(axis=2)
    # amax / 6 is not a float32 in general: compare with the cast of its float32 rounding, which
    # cannot cross an e4m3 tie (amax has 8 significant bits, so amax / 6 is never within 2^-24 of
    # one unless it is one)
    assert np.array_equal(rec[:, 256:], _torch_e4m3((amax / 6.0).astype(np.float32)))
    back = dequant_fp4_records(rec).reshape(64, 32, 16)
    sc = E4M3[rec[:, 256:]][:, :, None]
    y = np.abs(x.reshape(64, 32, 16) / sc)
    # half the gap between neighbouring e2m1 magnitudes around y (0.25 below 2, 0.5 up to 4, 1 to 6),
    # plus the saturation when the rounded scale is below amax / 6
    half_gap = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    over = np.maximum(y - 6, 0)
    assert np.all(np.abs(back - x.reshape(64, 32, 16)) <= (half_gap + over) * sc + 1e-300)


def test_encoders_agree_with_the_synthetic_cache_encoder():
    """The seeded workloads encode with torch's cast and a midpoint search; the oracle with
    nearest-value tables. Different code, the same records (up to the sign of zero, which the
    workloads drop for fp4)."""
    from workloads import encode_fp4_records as w_fp4, encode_fp8_records as w_fp8
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((256, 512)) * np.exp2(rng.uniform(-4, 4, (256, 16, 1)))
              .repeat(32, axis=2).reshape(256, 512))
    assert np.array_equal(encode_fp8_records(x), w_fp8(x.astype(np.float32)))
    a, b = encode_fp4_records(x), w_fp4(x.astype(np.float32))
    lo = lambda r: np.where(r & 0x0F == 8, r & 0xF0, r)
    hi = lambda r: np.where(r & 0xF0 == 0x80, r & 0x0F, r)
    assert np.array_equal(hi(lo(a[:, :256])), hi(lo(b[:, :256])))
    assert np.array_equal(a[:, 256:], b[:, 256:])
