"""Per-token record encoder (the cache writer), in float64.

Test infrastructure (see the package docstring): never used by the product path.

The pages fix what a record holds and where (page "flops/flashmla-decode-fp8-fp4-kv", section
"Arithmetic intensity"; page "deepseek-ai/FlashMLA", section "Key technical details"):

* fp8 record, 528 bytes: 512 float8_e4m3 values, then 16 float8_e8m0 scales, one per 32 consecutive
  values;
* fp4 record, 288 bytes: 256 bytes of e2m1, two values per byte with the even index in the low
  nibble, then 32 float8_e4m3 scales, one per 16 values.

They do not say how a writer picks the scales. This package reads that as follows (the plainest rule
that makes every block representable, and the one the synthetic caches use):

* fp8 block of 32 values x with a = max |x|: the scale is the smallest power of two 2^k with
  a <= 448 * 2^k, i.e. k = ceil(log2(a / 448)), clipped to the e8m0 range [-127, 127]; an all-zero
  block takes k = 0. The scale byte is k + 127 and each value is stored as the e4m3 value nearest to
  x / 2^k (ties to the even code). |x / 2^k| <= 448 by the choice of k, so nothing saturates.
* fp4 block of 16 values: the scale is the e4m3 value nearest to a / 6 (ties to the even code,
  saturating at 448); when that is 0 (an all-zero or vanishingly small block) the scale 1.0 is
  stored instead. Each value is stored as the e2m1 value nearest to x / scale (ties to the even
  code), saturating at +-6.
* Rounding keeps the sign, so a negative value that rounds to zero is stored as negative zero.

Inputs are finite (bfloat16 values in the tests); the element tables come from formats.py.
"""
import numpy as np

from .formats import E2M1, E4M3, FP4_RECORD_BYTES, FP8_RECORD_BYTES, HEAD_DIM

_E4M3_POS = E4M3[:0x7F]             # codes 0x00..0x7E: 0 and the positive finite values, ascending
_E2M1_POS = E2M1[:8]                 # codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6


def _nearest_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table entry nearest to each magnitude (table ascending, every entry's code its
    index); on a tie the even index wins. Magnitudes beyond the last entry take the last entry."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, mag, side="left"), 1, len(table) - 1)
    lo = hi - 1
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= table[-1], len(table) - 1, code)
    return code.astype(np.uint8)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code of each value (ties to even, saturating at +-448, sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_code(np.abs(x), _E4M3_POS)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code of each value (ties to even, saturating at +-6, sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_code(np.abs(x), _E2M1_POS)
    return code | (np.signbit(x).astype(np.uint8) << 3)


def fp8_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """k = ceil(log2(amax / 448)) clipped to [-127, 127]; 0 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        k = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0.0)
    return np.clip(k, -127, 127).astype(np.int64)


def encode_fp8_records(x: np.ndarray) -> np.ndarray:
    """[n, 512] values -> [n, 528] uint8 fp8 records."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    n = x.shape[0]
    blocks = x.reshape(n, 16, 32)
    k = fp8_scale_exponent(np.abs(blocks).max(axis=2))               # [n, 16]
    y = blocks / np.exp2(k)[:, :, None]                              # exact: a power of two
    rec = np.empty((n, FP8_RECORD_BYTES), dtype=np.uint8)
    rec[:, :HEAD_DIM] = e4m3_encode(y).reshape(n, HEAD_DIM)
    rec[:, HEAD_DIM:] = (k + 127).astype(np.uint8)
    return rec


def encode_fp4_records(x: np.ndarray) -> np.ndarray:
    """[n, 512] values -> [n, 288] uint8 fp4 records."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    n = x.shape[0]
    blocks = x.reshape(n, 32, 16)
    sc_code = e4m3_encode(np.abs(blocks).max(axis=2) / 6.0)          # [n, 32], never negative
    sc_code = np.where(E4M3[sc_code] == 0, np.uint8(0x38), sc_code)  # scale 1.0 for a zero scale
    codes = e2m1_encode(blocks / E4M3[sc_code][:, :, None]).reshape(n, HEAD_DIM)
    rec = np.empty((n, FP4_RECORD_BYTES), dtype=np.uint8)
    rec[:, :HEAD_DIM // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    rec[:, HEAD_DIM // 2:] = sc_code
    return rec
