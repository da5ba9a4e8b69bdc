"""Element decode tables and per-token record dequantisation, in float64.

Test infrastructure (see the package docstring): never used by the product path.

Record layouts, from page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity":

* fp8 record, 528 bytes: 512 float8_e4m3 values covering all 512 latent dims, then 16 float8_e8m0
  scales, one per 32 consecutive values (scale j covers dims 32j .. 32j+31).
* fp4 record, 288 bytes: 256 bytes of e2m1 holding two values per byte with the even index in the low
  nibble, then 32 float8_e4m3 scales, one per 16 values (scale j covers dims 16j .. 16j+15).

Page "deepseek-ai/FlashMLA", section "Key technical details", fixes the order: raw quantized values
first, the per-token scale factors after them.

The element encodings are the ones those names denote: OCP 8-bit float E4M3 in its "FN" form (bias 7,
no infinities, S.1111.111 is NaN, largest finite 448), the OCP Microscaling E8M0 scale (value
2^(byte-127), byte 0xFF is NaN) and the OCP Microscaling E2M1 element (bias 1, values 0, 0.5, 1, 1.5,
2, 3, 4, 6 and their negatives). A value is element * scale, computed exactly in float64.
"""
import numpy as np

HEAD_DIM = 512
FP8_RECORD_BYTES = 528          # 512 data + 16 scales
FP4_RECORD_BYTES = 288          # 256 data + 32 scales
FP8_BLOCK = 32                  # values per e8m0 scale
FP4_BLOCK = 16                  # values per e4m3 scale


def _e4m3_value(code: int) -> float:
    """OCP E4M3 ("FN"): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                                   # subnormal: 0.mmm * 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def _e8m0_value(code: int) -> float:
    """OCP MX E8M0 scale: 2^(code-127); code 0xFF is NaN."""
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


def _e2m1_value(code: int) -> float:
    """OCP MX E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:                                   # subnormal: 0.m * 2^(1-1)
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0 = np.array([_e8m0_value(c) for c in range(256)], dtype=np.float64)
E2M1 = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: a bfloat16 is the upper 16 bits of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def dequant_fp8_records(records: np.ndarray) -> np.ndarray:
    """[n, 528] uint8 fp8 records -> [n, 512] float64: x[i] = E4M3[rec[i]] * E8M0[rec[512 + i // 32]]."""
    rec = np.asarray(records, dtype=np.uint8).reshape(-1, FP8_RECORD_BYTES)
    data = E4M3[rec[:, :HEAD_DIM]]                                  # [n, 512]
    scales = E8M0[rec[:, HEAD_DIM:]]                                # [n, 16]
    return data * np.repeat(scales, FP8_BLOCK, axis=1)


def dequant_fp4_records(records: np.ndarray) -> np.ndarray:
    """[n, 288] uint8 fp4 records -> [n, 512] float64.

    Value i sits in byte i // 2, low nibble when i is even and high nibble when i is odd; its scale is
    the e4m3 byte 256 + i // 16.
    """
    rec = np.asarray(records, dtype=np.uint8).reshape(-1, FP4_RECORD_BYTES)
    packed = rec[:, :HEAD_DIM // 2]                                 # [n, 256]
    codes = np.empty((rec.shape[0], HEAD_DIM), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    scales = E4M3[rec[:, HEAD_DIM // 2:]]                           # [n, 32]
    return E2M1[codes] * np.repeat(scales, FP4_BLOCK, axis=1)
