"""Pins for the oracle's element tables and record dequant (CPU only).

Tables are checked against torch's own float8 decoders (a library routine independent of the oracle's
bit-field formulas), against the OCP MX E2M1 table fixture, and against hand-built records whose values
follow from the record layout on page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity".
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import (E2M1, E4M3, E8M0, bf16_bits_to_f64, dequant_fp4_records,
                    dequant_fp8_records)


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | ((a == b) & (np.signbit(a) == np.signbit(b)))))


def test_e4m3_table_matches_torch_decoder():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(E4M3, ref)


def test_e8m0_table_matches_torch_decoder():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(E8M0, ref)


def test_e4m3_spot_values():
    # OCP E4M3 FN: 0x38 = 1, 0x7E = 448 (largest), 0x01 = 2^-9 (smallest subnormal),
    # 0x08 = 2^-6 (smallest normal), 0x80 = -0, 0x7F / 0xFF = NaN, no infinities.
    assert E4M3[0x38] == 1.0 and E4M3[0x7E] == 448.0
    assert E4M3[0x01] == 2.0 ** -9 and E4M3[0x08] == 2.0 ** -6
    assert E4M3[0x80] == 0.0 and np.signbit(E4M3[0x80])
    assert math.isnan(E4M3[0x7F]) and math.isnan(E4M3[0xFF])
    assert np.all(np.isfinite(E4M3[~np.isnan(E4M3)]))
    assert np.nanmax(E4M3) == 448.0


def test_e8m0_spot_values():
    assert E8M0[0x7F] == 1.0 and E8M0[0x80] == 2.0 and E8M0[0x00] == 2.0 ** -127
    assert E8M0[0xFE] == 2.0 ** 127 and math.isnan(E8M0[0xFF])


def test_e2m1_table_matches_spec_fixture(golden_dir):
    rows = [ln.split() for ln in open(os.path.join(golden_dir, "e2m1_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        v = float(val)
        assert E2M1[int(code)] == v
        assert bool(np.signbit(E2M1[int(code)])) == (math.copysign(1.0, v) < 0)


def test_bf16_bits_match_torch():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert _same(bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


def test_fp8_record_scale_mapping_and_order():
    # fp8_a in tests/golden/record_layouts.txt
    rec = np.zeros(528, dtype=np.uint8)
    rec[:512] = 0x38
    rec[512:] = 0x7F + np.arange(16)
    x = dequant_fp8_records(rec[None])[0]
    assert np.array_equal(x, 2.0 ** (np.arange(512) // 32))
    # fp8_b
    rec = np.zeros(528, dtype=np.uint8)
    rec[:512:2] = 0x38
    rec[1:512:2] = 0xB8
    rec[512:] = 0x7E
    x = dequant_fp8_records(rec[None])[0]
    assert np.array_equal(x, 0.5 * (-1.0) ** np.arange(512))


def test_fp4_record_nibble_order():
    # fp4_a: even index in the low nibble
    rec = np.zeros(288, dtype=np.uint8)
    rec[:256] = 0x21
    rec[256:] = 0x38
    x = dequant_fp4_records(rec[None])[0]
    assert np.array_equal(x[0::2], np.full(256, 0.5)) and np.array_equal(x[1::2], np.full(256, 1.0))
    # fp4_c: sign bit of each nibble
    rec[:256] = 0x9F
    rec[256:] = 0x40
    x = dequant_fp4_records(rec[None])[0]
    assert np.array_equal(x[0::2], np.full(256, -12.0)) and np.array_equal(x[1::2], np.full(256, -1.0))


def test_fp4_record_scale_mapping():
    # fp4_b: scale j is the e4m3 code of the integer (j % 16) + 1 (codes from torch's encoder)
    rec = np.zeros(288, dtype=np.uint8)
    rec[:256] = 0x22
    rec[256:] = (torch.arange(32, dtype=torch.float32) % 16 + 1).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    x = dequant_fp4_records(rec[None])[0]
    assert np.array_equal(x, ((np.arange(512) // 16) % 16 + 1).astype(np.float64))


def test_dequant_is_exact_in_bfloat16_for_the_normal_scale_range():
    # Every e4m3 value times 2^(b-127) for b in [3, 246] has at most 4 significant bits and an
    # exponent inside bfloat16's range (subnormals included), so bfloat16 holds it exactly; the
    # device dequant is therefore compared bit-for-bit in that range.
    vals = E4M3[~np.isnan(E4M3)]
    for b in (3, 10, 64, 127, 200, 246):
        x = vals * 2.0 ** (b - 127)
        xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(x, xb)
    x = np.outer(E2M1, E4M3[~np.isnan(E4M3)]).ravel()
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(x, xb)
