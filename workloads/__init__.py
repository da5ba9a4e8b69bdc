"""Seeded synthetic decode workloads shared by the oracle tests, the GPU tests and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers and encodes them into the
cache byte formats (the decode side of those formats lives, independently, in the oracle and in the
HIP kernels). Encoding uses torch's own float8_e4m3fn cast; the e2m1 encoder is a nearest-value search.

Shapes follow the pages' DeepSeek decode setting (page "flops/flashmla-decode-fp8-fp4-kv"): a 512-dim
latent per token, 528-byte fp8 records, optional 288-byte fp4 "extra" records, a paged pool of 64-token
blocks addressed through a random block table, and per-row index lists of flat physical token ids
(physical_block * 64 + offset) with -1 for ignored entries.

Recipe (stated once, reused everywhere):
* q: float32 N(0,1) rounded to bfloat16.
* cache values: N(0,1) per element ("normal"), or N(0,1) * 2^u with u ~ U(-4, 4) drawn once per
  32-value block ("spread"). fp8 records: per 32 values, e8m0 scale 2^ceil(log2(amax / 448)), data
  = e4m3(x / scale) by round-to-nearest-even. fp4 records: per 16 values, e4m3 scale = e4m3(amax / 6),
  data = nearest e2m1 of x / scale (ties to the even code, saturating at 6).
* only selected records are encoded; every other record is filled with a poison pattern whose decoded
  values are huge, so a stray gather breaks parity at once.
* indices: per row, distinct logical positions drawn uniformly from the row's sequence (or every
  position in order), mapped through the block table; then -1 entries by the configured rule.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 512
BLOCK = 64
FP8_REC = 528
FP4_REC = 288
POISON_FP8 = (0x77, 0xF0)        # data byte, scale byte
POISON_FP4 = (0x77, 0x7E)


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    seq_len_q: int
    h_q: int
    topk: int
    tokens_per_seq: int
    extra_topk: int = 0
    extra_tokens_per_seq: int = 0
    values: str = "normal"            # "normal" | "spread"
    neg: str = "none"                 # "none" | "frac5" | "tail10" | "all"
    order: str = "random"             # "random" | "dense" (every position in order)
    softmax_scale: float = 1.0 / math.sqrt(HEAD_DIM)

    @property
    def rows(self) -> int:
        return self.batch * self.seq_len_q


# The five workloads of the decode benchmark family, by number.
CONFIGS = {
    0: Spec("tiny", 1, 1, 16, 128, 4096, neg="frac5"),
    1: Spec("mid", 32, 1, 64, 2048, 32768),
    2: Spec("headline", 128, 2, 128, 2048, 65536, values="spread", neg="tail10"),
    3: Spec("mixed", 64, 1, 64, 2048, 32768, extra_topk=512, extra_tokens_per_seq=8192),
    4: Spec("long", 8, 1, 128, 131072, 131072, order="dense"),
}


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def encode_fp8_records(x: np.ndarray) -> np.ndarray:
    """[n, 512] float values -> [n, 528] uint8 records (data, then 16 e8m0 scales)."""
    n = x.shape[0]
    blocks = np.asarray(x, dtype=np.float32).reshape(n, 16, 32)
    amax = np.abs(blocks).max(axis=2).astype(np.float64)
    with np.errstate(divide="ignore"):
        k = np.where(amax > 0, np.ceil(np.log2(amax / 448.0)), 0.0)
    k = np.clip(k, -127, 127).astype(np.int32)
    scaled = (blocks.astype(np.float64) / np.exp2(k)[:, :, None]).astype(np.float32)
    codes = torch.from_numpy(scaled.reshape(n, HEAD_DIM)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    out = np.empty((n, FP8_REC), dtype=np.uint8)
    out[:, :HEAD_DIM] = codes
    out[:, HEAD_DIM:] = (k + 127).astype(np.uint8)
    return out


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])   # midpoints between magnitudes


def _e2m1_codes(y: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code of each value (ties to the even code, magnitudes saturate at 6)."""
    mag = np.abs(y)
    code = np.searchsorted(_E2M1_MID, mag, side="left")            # midpoints strictly below
    tie = (code < 7) & (mag == _E2M1_MID[np.minimum(code, 6)])
    code = (code + (tie & (code % 2 == 1))).astype(np.uint8)
    sign = (np.signbit(y) & (code > 0)).astype(np.uint8)
    return code | (sign << 3)


def encode_fp4_records(x: np.ndarray) -> np.ndarray:
    """[n, 512] float values -> [n, 288] uint8 records (packed e2m1, then 32 e4m3 scales)."""
    n = x.shape[0]
    blocks = np.asarray(x, dtype=np.float32).reshape(n, 32, 16)
    amax = np.abs(blocks).max(axis=2)
    sc_codes = torch.from_numpy((amax / 6.0).astype(np.float32)).to(torch.float8_e4m3fn)
    sc_vals = sc_codes.to(torch.float64).numpy()
    sc_codes = sc_codes.view(torch.uint8).numpy().copy()
    zero = sc_vals == 0
    sc_codes[zero] = 0x38                                          # scale 1.0 for all-zero blocks
    sc_vals = np.where(zero, 1.0, sc_vals)
    codes = _e2m1_codes(blocks.astype(np.float64) / sc_vals[:, :, None]).reshape(n, HEAD_DIM)
    out = np.empty((n, FP4_REC), dtype=np.uint8)
    out[:, :HEAD_DIM // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, HEAD_DIM // 2:] = sc_codes
    return out


def _values(rng: np.random.Generator, n: int, mode: str) -> np.ndarray:
    x = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    if mode == "spread":
        u = rng.uniform(-4.0, 4.0, size=(n, 16)).astype(np.float32)
        x = (x.reshape(n, 16, 32) * np.exp2(u)[:, :, None]).reshape(n, HEAD_DIM)
    return x


def _poison_pool(n: int, rec: int, pattern) -> np.ndarray:
    pool = np.empty((n, rec), dtype=np.uint8)
    data_bytes = HEAD_DIM if rec == FP8_REC else HEAD_DIM // 2
    pool[:, :data_bytes] = pattern[0]
    pool[:, data_bytes:] = pattern[1]
    return pool


def _select(rng, spec_rows, batch, seq_len_q, topk, tokens_per_seq, order, table):
    """Per-row flat physical token ids [rows, topk] (before -1 masking)."""
    rows = batch * seq_len_q
    out = np.empty((rows, topk), dtype=np.int64)
    for r in range(rows):
        b = r // seq_len_q
        if order == "dense":
            pos = np.arange(topk, dtype=np.int64)
        else:
            pos = rng.choice(tokens_per_seq, size=topk, replace=False).astype(np.int64)
        out[r] = table[b, pos // BLOCK] * BLOCK + pos % BLOCK
    return out


def _apply_neg(rng, idx: np.ndarray, mode: str) -> np.ndarray:
    rows, topk = idx.shape
    idx = idx.copy()
    if mode == "frac5":
        k = int(round(0.05 * topk))
        for r in range(rows):
            idx[r, rng.choice(topk, size=k, replace=False)] = -1
    elif mode == "tail10":
        for r in range(rows):
            k = int(math.floor(rng.uniform() * 0.10 * topk))
            if k:
                idx[r, topk - k:] = -1
    elif mode == "all":
        idx[:] = -1
    return idx


def make_workload(spec: Spec | int, seed: int | None = None, encode_chunk: int = 65536) -> dict:
    """Build one workload. Returns numpy arrays:

    q_bits uint16 [B, S, H, 512]; k_cache uint8 [N, 528]; indices int32 [B, S, topk];
    extra_k_cache uint8 [N2, 288] or None; extra_indices int32 [B, S, extra_topk] or None;
    softmax_scale float; spec.
    """
    if isinstance(spec, int):
        if seed is None:
            seed = 1000 + spec
        spec = CONFIGS[spec]
    if seed is None:
        seed = 1234
    ss = np.random.SeedSequence(seed)
    r_q, r_cache, r_table, r_idx, r_xcache, r_xtable, r_xidx = [np.random.default_rng(s)
                                                                 for s in ss.spawn(7)]
    b_, s_, h_ = spec.batch, spec.seq_len_q, spec.h_q
    q_bits = _bf16_bits(r_q.standard_normal((b_, s_, h_, HEAD_DIM), dtype=np.float32))

    def build(rng_c, rng_t, rng_i, topk, per_seq, rec, pattern, encoder, neg):
        blocks_per_seq = -(-per_seq // BLOCK)
        nblocks = b_ * blocks_per_seq
        table = rng_t.permutation(nblocks).reshape(b_, blocks_per_seq)
        phys = _select(rng_i, None, b_, s_, topk, per_seq, spec.order, table)
        idx = _apply_neg(rng_i, phys, neg)
        pool = _poison_pool(nblocks * BLOCK, rec, pattern)
        sel = np.unique(idx[idx >= 0])
        for a in range(0, sel.size, encode_chunk):
            part = sel[a:a + encode_chunk]
            pool[part] = encoder(_values(rng_c, part.size, spec.values))
        return pool, idx.astype(np.int32).reshape(b_, s_, topk)

    k_cache, indices = build(r_cache, r_table, r_idx, spec.topk, spec.tokens_per_seq, FP8_REC,
                             POISON_FP8, encode_fp8_records, spec.neg)
    extra_k_cache = extra_indices = None
    if spec.extra_topk:
        extra_k_cache, extra_indices = build(r_xcache, r_xtable, r_xidx, spec.extra_topk,
                                             spec.extra_tokens_per_seq, FP4_REC, POISON_FP4,
                                             encode_fp4_records, spec.neg)
    return dict(spec=spec, q_bits=q_bits, k_cache=k_cache, indices=indices,
                extra_k_cache=extra_k_cache, extra_indices=extra_indices,
                softmax_scale=spec.softmax_scale)


def add_index_set(w: dict, seed: int, encode_chunk: int = 65536) -> np.ndarray:
    """Draw another fp8 index set for the same rows and shapes as workload `w` (new distinct positions,
    same -1 rule), encode the newly selected records into w["k_cache"] in place, and return the
    int32 [B, S, topk] indices. Used to give successive benchmark steps different tokens."""
    spec = w["spec"]
    b_, s_ = spec.batch, spec.seq_len_q
    rng_t, rng_i, rng_c = [np.random.default_rng(x) for x in np.random.SeedSequence(seed).spawn(3)]
    blocks_per_seq = -(-spec.tokens_per_seq // BLOCK)
    table = rng_t.permutation(b_ * blocks_per_seq).reshape(b_, blocks_per_seq)
    phys = _select(rng_i, None, b_, s_, spec.topk, spec.tokens_per_seq, spec.order, table)
    idx = _apply_neg(rng_i, phys, spec.neg)
    pool = w["k_cache"]
    sel = np.unique(idx[idx >= 0])
    for a in range(0, sel.size, encode_chunk):
        part = sel[a:a + encode_chunk]
        pool[part] = encode_fp8_records(_values(rng_c, part.size, spec.values))
    return idx.astype(np.int32).reshape(b_, s_, spec.topk)


def add_extra_index_set(w: dict, seed: int, encode_chunk: int = 65536) -> np.ndarray:
    """The same as add_index_set for the fp4 extra cache of workload `w`: new distinct positions in
    each row's extra sequence, newly selected fp4 records encoded into w["extra_k_cache"] in place.
    Returns the int32 [B, S, extra_topk] indices."""
    spec = w["spec"]
    b_, s_ = spec.batch, spec.seq_len_q
    rng_t, rng_i, rng_c = [np.random.default_rng(x) for x in np.random.SeedSequence(seed).spawn(3)]
    blocks_per_seq = -(-spec.extra_tokens_per_seq // BLOCK)
    table = rng_t.permutation(b_ * blocks_per_seq).reshape(b_, blocks_per_seq)
    phys = _select(rng_i, None, b_, s_, spec.extra_topk, spec.extra_tokens_per_seq, spec.order, table)
    idx = _apply_neg(rng_i, phys, spec.neg)
    pool = w["extra_k_cache"]
    sel = np.unique(idx[idx >= 0])
    for a in range(0, sel.size, encode_chunk):
        part = sel[a:a + encode_chunk]
        pool[part] = encode_fp4_records(_values(rng_c, part.size, spec.values))
    return idx.astype(np.int32).reshape(b_, s_, spec.extra_topk)
