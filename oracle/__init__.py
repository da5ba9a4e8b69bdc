"""CPU oracle for token-sparse MLA decode over a quantized, paged latent KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library (``sparse_mla_decode_get_amd``) and imports nothing from it.

Everything here is plain, slow and float64, written from the pages' own statements:

* ``formats``   -- element decode tables (OCP e4m3 / e8m0 / e2m1) and per-token record dequant
                   (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity";
                   page "deepseek-ai/FlashMLA", section "Key technical details").
* ``attention`` -- softmax attention of each query row over its selected tokens, the split form and
                   the log-sum-exp merge of splits (page "flops/flashmla-decode-fp8-fp4-kv",
                   section "Workarounds"; page "deepseek-ai/FlashMLA", section "How to use it").
* ``metadata``  -- the tile-scheduler partition computed once before the decode loop (same sections).
                   The pages give only its existence, so its content is this package's own spec.
* ``encode``    -- the cache writer: bf16 latents -> 528 B fp8 / 288 B fp4 records (page
                   "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic intensity"); the pages
                   fix the layout, the scale choice is this package's reading (see that module).

Parity status: every function is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
against library decoders, closed forms, invariants and hand-derived fixtures under ``tests/golden/``.
"""
from .formats import (E2M1, E4M3, E8M0, FP4_RECORD_BYTES, FP8_RECORD_BYTES, HEAD_DIM,
                      bf16_bits_to_f64, dequant_fp4_records, dequant_fp8_records)
from .attention import (oracle_combine, oracle_decode, oracle_decode_rows, oracle_split_decode,
                        row_token_lists)
from .metadata import TILE_TOKENS, oracle_metadata, part_count, tiles_per_row
from .encode import (e2m1_encode, e4m3_encode, encode_fp4_records, encode_fp8_records,
                     fp8_scale_exponent)

__all__ = [
    "E2M1", "E4M3", "E8M0", "FP4_RECORD_BYTES", "FP8_RECORD_BYTES", "HEAD_DIM", "TILE_TOKENS",
    "bf16_bits_to_f64", "dequant_fp4_records", "dequant_fp8_records", "oracle_combine",
    "oracle_decode", "oracle_decode_rows", "oracle_metadata", "oracle_split_decode", "part_count",
    "row_token_lists", "tiles_per_row", "e2m1_encode", "e4m3_encode", "encode_fp4_records",
    "encode_fp8_records", "fp8_scale_exponent",
]
