"""GPU parity on inputs built to reach the softmax's rarely taken paths.

The two-half 64-head kernel (h_q <= 64, short parts) keeps a running maximum per head and rescales
its output accumulator only when a later sub-tile's maximum exceeds it by more than 8 (log2 units);
the single-stream 64-head kernel (h_q <= 64, parts of 6 or more sub-tiles) and the 128-head kernel
take probabilities against the first live sub-tile's maximum and compute a segment again when a
later score exceeds that reference by more than 64. Random N(0,1) caches reach neither path, so
these inputs control the scores:

* every head's query is a scaled copy of one base vector b plus small noise, so a latent along b
  scores nearly the same (chosen) value in every head, growing with the head index;
* "moderate": the row's first 64 tokens (the first sub-tile of each half of the 64-head kernel) and
  a background of other tokens have small latents (scores near 0); one "spike" token per half of the
  later sub-tiles lies along b and scores 10-20 log2 units: the running maximum grows by more than
  8 while the first tokens keep about 1% of the softmax weight in the low heads, so a wrong rescale
  factor shows in the output;
* "extreme": later tokens' latents are 256 times larger (e8m0 scale bytes + 8, or fp4 e4m3 scale
  exponents + 8), so scores grow by far more than 64 log2 units past the first sub-tile.

Each case asserts from the oracle's own scores that the growth it is meant to produce is there,
then compares the HIP path with the oracle at the usual tolerances.
"""
import math

import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import bf16_bits_to_f64, dequant_fp4_records, dequant_fp8_records, oracle_decode
from workloads import Spec, encode_fp4_records, encode_fp8_records, make_workload
from tests.gpu_helpers import check_rows, to_dev

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _row_latents(w, r):
    """Dequantized latents of row r in selection order (fp8 list, then fp4 list) and the position
    of each in its unit sequence (fp8 slot p -> sub-tile p // 32; fp4 slot p -> after the fp8
    units)."""
    spec = w["spec"]
    idx = w["indices"].reshape(spec.rows, -1)[r]
    lat, sub = [], []
    tiles_k = -(-spec.topk // 64)
    for p, t in enumerate(idx):
        if t >= 0:
            lat.append(dequant_fp8_records(w["k_cache"][t][None])[0])
            sub.append(p // 32)
    if spec.extra_topk:
        xidx = w["extra_indices"].reshape(spec.rows, -1)[r]
        for p, t in enumerate(xidx):
            if t >= 0:
                lat.append(dequant_fp4_records(w["extra_k_cache"][t][None])[0])
                sub.append(2 * tiles_k + p // 32)
    return np.array(lat), np.array(sub)


def _scores_log2(w, r):
    spec = w["spec"]
    q = bf16_bits_to_f64(w["q_bits"]).reshape(spec.rows, spec.h_q, 512)[r]
    lat, sub = _row_latents(w, r)
    return spec.softmax_scale * (q @ lat.T) * LOG2E, sub      # [H, n] in log2 units


def _controlled(spec, seed, mode):
    """Workload of `spec` whose query and selected latents follow the module docstring."""
    w = make_workload(spec, seed=seed)
    rng = np.random.default_rng(seed + 99)
    rows, h = spec.rows, spec.h_q
    q = np.empty((rows, h, 512), np.float32)
    tiles_k = -(-spec.topk // 64)
    for r in range(rows):
        b = rng.standard_normal(512).astype(np.float32)
        b /= np.linalg.norm(b) / math.sqrt(512)           # |b|^2 = 512
        grow = 1.0 + np.arange(h, dtype=np.float32)[:, None] / max(h - 1, 1)
        q[r] = grow * b[None, :] + 0.25 * rng.standard_normal((h, 512)).astype(np.float32)
        unit_b = b / np.linalg.norm(b)
        # one spike latent scoring about 10.5 log2 units in head 0 (about 21 in the last head)
        alpha = 10.5 / LOG2E / (spec.softmax_scale * math.sqrt(512))
        idx = w["indices"].reshape(rows, -1)[r]
        fp8_vals = 0.05 * rng.standard_normal((idx.size, 512)).astype(np.float32)
        if mode == "moderate" and spec.extra_topk == 0:
            # the first live sub-tile of each half is 0 and 1; spikes in sub-tiles 2 and 3
            for s in (2, 3):
                if s * 32 < idx.size:
                    fp8_vals[s * 32 + 5] = alpha * unit_b
        sel = idx >= 0
        w["k_cache"][idx[sel]] = encode_fp8_records(fp8_vals[sel])
        if spec.extra_topk:
            xidx = w["extra_indices"].reshape(rows, -1)[r]
            fp4_vals = 0.05 * rng.standard_normal((xidx.size, 512)).astype(np.float32)
            if mode == "moderate":
                for s in (0, 1):                               # fp4 sub-tiles follow the fp8 ones
                    if s * 32 < xidx.size:
                        fp4_vals[s * 32 + 5] = alpha * unit_b
            xsel = xidx >= 0
            w["extra_k_cache"][xidx[xsel]] = encode_fp4_records(fp4_vals[xsel])
        if mode == "extreme":
            # every token past the first 64 entries of the fp8 list (the first sub-tile of either
            # half): values x 256
            later = np.unique(idx[64:][idx[64:] >= 0])
            later = np.setdiff1d(later, idx[:64])
            w["k_cache"][later, 512:] += 8
            if spec.extra_topk:
                xl = np.unique(xidx[xidx >= 0])
                sc = w["extra_k_cache"][xl, 256:].astype(np.int32)
                assert ((sc & 0x78) >> 3).max() + 8 <= 14          # e4m3 exponent stays finite
                w["extra_k_cache"][xl, 256:] = (sc + (8 << 3)).astype(np.uint8)
    w["q_bits"] = _bf16_bits(q).reshape(spec.batch, spec.seq_len_q, h, 512)
    return w


CASES = [
    # (name, h_q, topk, extra_topk, mode)
    ("h16_fp8_moderate", 16, 256, 0, "moderate"),
    ("h64_fp8_moderate", 64, 256, 0, "moderate"),
    ("h16_fp4_moderate", 16, 256, 96, "moderate"),
    ("h64_fp4_moderate", 64, 256, 96, "moderate"),
    ("h128_fp8_moderate", 128, 256, 0, "moderate"),
    ("h128_fp4_moderate", 128, 256, 96, "moderate"),
    ("h16_fp8_extreme", 16, 256, 0, "extreme"),
    ("h64_fp8_extreme", 64, 256, 0, "extreme"),
    ("h64_fp4_extreme", 64, 256, 96, "extreme"),
    ("h128_fp8_extreme", 128, 256, 0, "extreme"),
    ("h128_fp4_extreme", 128, 256, 96, "extreme"),
    # rows of 2 fp8 and 2 fp4 sub-tiles: whole rows also run the two-half kernel, whose running
    # maximum then grows inside the fp4 sub-tiles
    ("h16_fp4_moderate_short", 16, 64, 64, "moderate"),
    ("h64_fp4_moderate_short", 64, 64, 64, "moderate"),
    ("h64_fp4_extreme_short", 64, 64, 64, "extreme"),
]


@pytest.mark.parametrize("name,h_q,topk,extra,mode", CASES, ids=[c[0] for c in CASES])
def test_score_growth_reaches_the_rescale_paths(name, h_q, topk, extra, mode):
    # one query row per sequence, so that no two rows share (and rewrite) a token's record
    spec = Spec(name, 4, 1, h_q, topk, 4096, extra_topk=extra,
                extra_tokens_per_seq=1024 if extra else 0)
    w = _controlled(spec, seed=61 + h_q + extra, mode=mode)
    rows = spec.rows
    # what the inputs are meant to produce, read from the oracle's own scores (one part per row,
    # so every row is one segment starting at its first sub-tile)
    for r in range(rows):
        s, sub = _scores_log2(w, r)
        if h_q <= 64:
            # halves: sub-tiles of even / odd index; growth of each half's maximum past its first
            for half in (0, 1):
                mine = sub % 2 == half
                first = mine & (sub == sub[mine].min())
                growth = s[:, mine].max(axis=1) - s[:, first].max(axis=1)
                assert (growth > 8).sum() >= h_q // 2, f"{name} row {r}: too little growth"
            if mode == "moderate":
                p = np.exp2(s - s.max(axis=1, keepdims=True))
                f_first = p[:, sub < 2].sum(axis=1) / p.sum(axis=1)
                assert f_first.max() > 0.01, f"{name} row {r}: first tokens carry no weight"
        else:
            first = sub == sub.min()
            growth = s.max(axis=1) - s[:, first].max(axis=1)
            if mode == "extreme":
                assert growth.max() > 64, f"{name} row {r}: growth {growth.max():.1f} <= 64"
    d = to_dev(w)
    # h_q <= 64: one part per row of 8 fp8 sub-tiles (and 4 fp4 ones with the extra cache) runs
    # the single-stream kernel, of 4 sub-tiles (the short rows) and three parts per row the
    # two-half kernel
    md = mla.get_metadata(spec.batch, spec.seq_len_q, h_q, spec.topk, extra, num_parts=rows)
    out, lse = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md,
                                 d.get("extra_k_cache"), d.get("extra_indices"))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"],
                                     w["extra_k_cache"], w["extra_indices"])
    check_rows(out, lse, ref_out, ref_lse, name)
    # and under the default schedule (rows split over parts, each part's segment restarting the
    # running maximum)
    md2 = mla.get_metadata(spec.batch, spec.seq_len_q, h_q, spec.topk, extra, num_parts=3 * rows)
    out2, lse2 = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md2,
                                   d.get("extra_k_cache"), d.get("extra_indices"))
    torch.cuda.synchronize()
    check_rows(out2, lse2, ref_out, ref_lse, name + "/split")


STREAM_CASES = [
    ("h16_fp8_extreme_stream", 16, "extreme"),
    ("h64_fp8_extreme_stream", 64, "extreme"),
    ("h64_fp8_moderate_stream", 64, "moderate"),
]


@pytest.mark.parametrize("name,h_q,mode", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_score_growth_single_stream_64_head_kernel(name, h_q, mode):
    """The single-stream 64-head kernel (parts of at least 6 sub-tiles) takes
    probabilities against each head's first live sub-tile like the 128-head kernel: "extreme" rows
    grow by more than 64 log2 units past it, which forces the second pass."""
    spec = Spec(name, 4, 1, h_q, 1024, 8192)
    w = _controlled(spec, seed=71 + h_q, mode=mode)
    for r in range(spec.rows):
        s, sub = _scores_log2(w, r)
        first = sub == sub.min()
        growth = s.max(axis=1) - s[:, first].max(axis=1)
        if mode == "extreme":
            assert growth.max() > 64, f"{name} row {r}: growth {growth.max():.1f} <= 64"
        else:
            assert growth.max() > 8, f"{name} row {r}: growth {growth.max():.1f} <= 8"
    d = to_dev(w)
    ref_out, ref_lse = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"])
    # one part per row (32 sub-tiles), then two (16 sub-tiles each)
    for parts in (spec.rows, 2 * spec.rows):
        md = mla.get_metadata(spec.batch, spec.seq_len_q, h_q, spec.topk, 0, num_parts=parts)
        out, lse = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md)
        torch.cuda.synchronize()
        check_rows(out, lse, ref_out, ref_lse, f"{name}/{parts} parts")
