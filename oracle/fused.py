"""Fused decode: Q-norm, RoPE, sparse attention, conjugate RoPE on the output, cast to FP8; float64.

Test infrastructure (see the package docstring): never used by the product path.

The pages name the steps and their order (page "deepseek-ai/FlashMLA", section "What it is": one
kernel combining Q-norm, RoPE, the core attention, the conjugate RoPE on the output side and the
final cast to FP8; section "How to use it": the decode call of that kernel returns FP8 outputs for a
downstream FP8 einsum). They leave the details open; this package reads them as follows:

* Q-norm: RMSNorm of each head's 512-dim query row with a learned weight w[512]:
  q' = q / sqrt(mean(q^2) + eps) * w.
* RoPE: the last 64 of the 512 latent dims (448..511) carry the rotary part, as 32 interleaved pairs
  (448 + 2i, 449 + 2i); pair i of query row r is rotated by the angle whose cosine and sine the caller
  passes, cos[r, i] and sin[r, i] (the frequencies are the model's, not the kernel's):
  (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
* The normalised, rotated query enters QK^T as bfloat16 (nearest, ties to even), as the plain
  decode's query does; attention is then exactly oracle_decode's.
* Conjugate RoPE: the output's pairs are rotated back by the same angle:
  (y0, y1) -> (y0 cos + y1 sin, -y0 sin + y1 cos).
* FP8 cast: every (row, head) output row is stored as one of the pages' 528-byte fp8 records
  (512 e4m3 values, then 16 e8m0 scales, one per 32 values), encoded by encode.encode_fp8_records.
  A row with no valid entry has out = 0, i.e. an all-zero record with scale bytes 127.
"""
import numpy as np

from .attention import oracle_decode
from .encode import encode_fp8_records
from .formats import HEAD_DIM, bf16_bits_to_f64

ROPE_START = 448                 # first rotary dim
ROPE_PAIRS = 32


def rms_norm(q: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """q [..., 512] / sqrt(mean(q^2) + eps) * weight[512]."""
    q = np.asarray(q, dtype=np.float64)
    return q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps) * np.asarray(weight, np.float64)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, conjugate: bool = False) -> np.ndarray:
    """Rotate pairs (448 + 2i, 449 + 2i) of x [..., 512] by cos/sin [..., 32] (broadcast over the
    axes between); conjugate rotates by the opposite angle."""
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    x0 = x[..., ROPE_START::2]
    x1 = x[..., ROPE_START + 1::2]
    s = -sin if conjugate else sin
    y[..., ROPE_START::2] = x0 * cos - x1 * s
    y[..., ROPE_START + 1::2] = x0 * s + x1 * cos
    return y


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even): bfloat16 keeps 8 significant bits, so
    a normal x = m * 2^e with m in [1, 2) rounds to a multiple of 2^(e - 7); below 2^-126 the grid
    is 2^-133. Finite inputs within the bfloat16 range."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    step = np.exp2(np.maximum(e, -126.0) - 7.0)
    return np.where(mag > 0, np.round(x / step) * step, x)   # np.round: ties to even


def oracle_fused_decode(q_bits, norm_weight_bits, eps, rope_cos, rope_sin, k_cache, indices,
                        softmax_scale, extra_k_cache=None, extra_indices=None):
    """q_bits bf16 bits [B, S, H, 512] (the raw query), norm_weight_bits bf16 bits [512], rope_cos /
    rope_sin [B, S, 32] (as the kernel receives them, float32 values). Returns
    (records uint8 [B, S, H, 528], lse float64 [B, S, H], out_rotated float64 [B, S, H, 512]), the
    last being the exact output before the FP8 cast."""
    q = bf16_bits_to_f64(q_bits)
    w = bf16_bits_to_f64(norm_weight_bits)
    cos = np.asarray(rope_cos, dtype=np.float64)[:, :, None, :]       # broadcast over heads
    sin = np.asarray(rope_sin, dtype=np.float64)[:, :, None, :]
    q_in = round_bf16(rope(rms_norm(q, w, eps), cos, sin))
    out, lse = oracle_decode(q_in, k_cache, indices, softmax_scale, extra_k_cache, extra_indices)
    out_r = rope(out, cos, sin, conjugate=True)
    b, s, h, _ = out_r.shape
    rec = encode_fp8_records(out_r.reshape(-1, HEAD_DIM)).reshape(b, s, h, 528)
    return rec, lse, out_r
