"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Bit-exact: record dequantisation (in the exact bf16 range) and the tile-scheduler metadata.
Within tolerance (max |d out| <= 2e-2 max |ref| per row, |d lse| <= 1e-3): decode and merge, on
small shapes spanning several tiles with ragged tails and edge cases, and on every row of the
full-size workloads in the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import (E4M3, dequant_fp4_records, dequant_fp8_records, oracle_combine, oracle_decode,
                    oracle_decode_rows, oracle_metadata, oracle_split_decode)
from workloads import CONFIGS, Spec, make_workload
from tests.gpu_helpers import bf16_rne, bf16_to_f64, check_rows, to_dev

pytestmark = pytest.mark.gpu


def _decode(w, num_parts=0, min_tiles=1):
    d = to_dev(w)
    b, s, h, _ = d["q"].shape
    extra = d["extra_indices"].shape[2] if "extra_indices" in d else 0
    md = mla.get_metadata(b, s, h, d["indices"].shape[2], extra, num_parts, min_tiles)
    out, lse = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md,
                                 d.get("extra_k_cache"), d.get("extra_indices"))
    torch.cuda.synchronize()
    return out, lse, md


def _oracle(w):
    return oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"],
                         w["extra_k_cache"], w["extra_indices"])


# ----------------------------------------------------------------------------- dequant (bit-exact)

def test_fp8_dequant_bit_exact_over_the_exact_scale_range():
    recs = []
    for b in range(3, 247):
        r = np.empty(528, dtype=np.uint8)
        r[:512] = np.tile(np.arange(256, dtype=np.uint8), 2)
        r[512:] = b
        recs.append(r)
    recs = np.stack(recs)
    idx = torch.arange(len(recs), dtype=torch.int32, device="cuda")
    got = bf16_to_f64(mla.dequant_records(torch.from_numpy(recs).cuda(), 528, idx))
    ref = dequant_fp8_records(recs)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])           # exact: no rounding in this range


def test_fp8_dequant_edge_scales_round_to_nearest_and_nan():
    recs = []
    for b in (0, 1, 2, 247, 250, 254, 255):
        r = np.empty(528, dtype=np.uint8)
        r[:512] = np.tile(np.arange(256, dtype=np.uint8), 2)
        r[512:] = b
        recs.append(r)
    recs = np.stack(recs)
    idx = torch.arange(len(recs), dtype=torch.int32, device="cuda")
    got = bf16_to_f64(mla.dequant_records(torch.from_numpy(recs).cuda(), 528, idx))
    ref = bf16_rne(dequant_fp8_records(recs))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp4_dequant_bit_exact_all_codes_and_scales():
    recs = []
    for k in range(8):                                    # 8 records x 32 scales = all 256 e4m3 codes
        r = np.empty(288, dtype=np.uint8)
        r[:256] = np.arange(256, dtype=np.uint8)          # every (low, high) nibble pair
        r[256:] = np.arange(32 * k, 32 * k + 32, dtype=np.uint8)
        recs.append(r)
    recs = np.stack(recs)
    idx = torch.arange(len(recs), dtype=torch.int32, device="cuda")
    got = bf16_to_f64(mla.dequant_records(torch.from_numpy(recs).cuda(), 288, idx))
    ref = dequant_fp4_records(recs)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_dequant_gathers_by_index():
    rng = np.random.default_rng(0)
    recs = rng.integers(0, 256, size=(64, 528), dtype=np.uint8)
    recs[:, 512:] = rng.integers(100, 150, size=(64, 16))
    recs[:, :512][recs[:, :512] & 0x7F == 0x7F] = 0      # no NaN codes
    sel = np.array([5, 0, 63, 5, 17], dtype=np.int32)
    got = bf16_to_f64(mla.dequant_records(torch.from_numpy(recs).cuda(), 528,
                                          torch.from_numpy(sel).cuda()))
    assert np.array_equal(got, dequant_fp8_records(recs[sel]))


# ---------------------------------------------------------------------------- metadata (bit-exact)

@pytest.mark.parametrize("batch,seq,topk,extra,parts,min_tiles", [
    (1, 1, 128, 0, 256, 1), (128, 2, 2048, 0, 256, 1), (32, 1, 2048, 0, 512, 1),
    (64, 1, 2048, 512, 512, 1), (8, 1, 131072, 0, 256, 1), (3, 2, 150, 70, 7, 2), (5, 1, 64, 0, 3, 1),
    (2, 1, 0, 0, 4, 1), (1, 1, 2048, 0, 256, 1), (700, 3, 70, 0, 1000, 1), (1500, 1, 128, 0, 999, 3)])
def test_metadata_bit_exact(batch, seq, topk, extra, parts, min_tiles):
    md = mla.get_metadata(batch, seq, 64, topk, extra, parts, min_tiles)
    torch.cuda.synchronize()
    sched, split_ptr, p_eff = oracle_metadata(batch, seq, topk, extra, parts, min_tiles)
    assert md.num_parts == p_eff
    assert np.array_equal(md.sched.cpu().numpy(), sched)
    assert np.array_equal(md.split_ptr.cpu().numpy(), split_ptr)


# ----------------------------------------------------------------------------- decode (tolerance)

SMALL = [
    Spec("cfg0", 1, 1, 16, 128, 4096, neg="frac5"),
    Spec("h32_ragged", 2, 1, 32, 300, 4096, neg="frac5"),
    Spec("h64_sq2", 2, 2, 64, 257, 2048),
    Spec("h128_spread", 2, 2, 128, 200, 4096, values="spread", neg="tail10"),
    Spec("h128_topk1", 3, 1, 128, 1, 512),
    Spec("h100_masked_heads", 2, 1, 100, 96, 1024),
    Spec("h200_two_groups", 1, 2, 200, 130, 1024, neg="frac5"),
    Spec("h1", 2, 1, 1, 64, 512),
    Spec("all_ignored", 2, 1, 64, 100, 1024, neg="all"),
    Spec("mixed_fp4", 2, 1, 64, 130, 2048, extra_topk=70, extra_tokens_per_seq=1024),
    Spec("mixed_h128", 2, 2, 128, 64, 1024, extra_topk=200, extra_tokens_per_seq=1024,
         values="spread"),
    Spec("fp4_only_extra", 2, 1, 32, 0, 64, extra_topk=100, extra_tokens_per_seq=512),
    Spec("fp4_only_h128", 2, 1, 128, 0, 64, extra_topk=100, extra_tokens_per_seq=512),
    Spec("all_ignored_h128", 2, 1, 128, 300, 1024, neg="all"),
    Spec("h128_ragged_long", 1, 2, 128, 1000, 8192, neg="frac5"),
    Spec("h128_topk20", 2, 1, 128, 20, 512),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s.name for s in SMALL])
def test_decode_small_default_schedule(spec):
    w = make_workload(spec, seed=7)
    out, lse, _ = _decode(w)
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, spec.name)


@pytest.mark.parametrize("spec,parts,min_tiles", [
    (Spec("split_h128", 2, 1, 128, 2048, 8192), 7, 1),
    (Spec("split_h64", 3, 2, 64, 700, 4096, neg="tail10"), 5, 1),
    (Spec("split_mixed", 2, 1, 64, 300, 2048, extra_topk=150, extra_tokens_per_seq=1024), 9, 1),
    (Spec("split_h16", 1, 1, 16, 1000, 4096, neg="frac5"), 16, 1),
    (Spec("one_part", 3, 2, 128, 150, 2048), 1, 1),
    (Spec("split_empty_rows", 2, 1, 64, 500, 2048, neg="all"), 4, 1),
    # 64-head kernel with heads 40..63 of its group past h_q, and four parts of 9 units over six
    # rows of 6: each part runs several row segments (staging Q again at the start of every one)
    # and some rows are split
    (Spec("h40_multi_segment", 3, 2, 40, 333, 2048, neg="frac5"), 4, 1),
], ids=lambda x: x.name if isinstance(x, Spec) else str(x))
def test_decode_split_rows(spec, parts, min_tiles):
    w = make_workload(spec, seed=11)
    out, lse, md = _decode(w, num_parts=parts, min_tiles=min_tiles)
    if spec.name != "one_part":
        assert md.workspace is not None            # some row really is split
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, spec.name)


@pytest.mark.parametrize("parts", [0, 5, 23])
def test_decode_trailing_ignored_subtiles(parts):
    """Rows whose selections end in runs of -1 of every length relative to the 32-token sub-tile
    (live prefixes of 0, 1, 31, 32, 33, 95, 500 and all 1000 entries), one row with a fully ignored
    sub-tile inside its live part, under the default schedule and under splits that leave whole
    segments with no valid entry."""
    spec = Spec("trailing", 4, 2, 128, 1000, 4096)
    w = make_workload(spec, seed=31)
    idx = w["indices"].reshape(8, 1000)
    for r, n_live in enumerate([0, 1, 31, 32, 33, 95, 500, 1000]):
        idx[r, n_live:] = -1
    idx[6, 64:96] = -1                            # a whole sub-tile inside the live part
    idx[7, 999] = -1                              # the last entry ignored, the rest live
    out, lse, md = _decode(w, num_parts=parts)
    if parts:
        assert md.workspace is not None
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, f"trailing/{parts}")
    assert torch.all(lse[0, 0] == -math.inf)      # the row with no valid entry
    assert torch.all(out[0, 0] == 0)


def test_scores_growing_past_the_first_subtile():
    """Later tokens carry 2^8-times larger values, so scores grow by far more than 2^64 over the
    first 32 tokens' maximum: the decode must still match (a probability reference taken from the
    first tokens alone would overflow)."""
    spec = Spec("growth", 1, 1, 128, 300, 2048)
    w = make_workload(spec, seed=21)
    later = np.unique(w["indices"][0, 0, 32:])
    later = later[later >= 0]
    first = set(w["indices"][0, 0, :32].tolist())
    later = np.array([t for t in later if t not in first], dtype=np.int64)
    kc = w["k_cache"].copy()
    kc[later, 512:] += 8                          # e8m0 scale bytes: values x 256
    assert kc[later, 512:].max() <= 246
    w["k_cache"] = kc
    out, lse, _ = _decode(w)
    ref_out, ref_lse = _oracle(w)
    assert (ref_lse.max() - 0) > 40               # the scores really are large
    check_rows(out, lse, ref_out, ref_lse, spec.name)


def test_split_and_unsplit_agree_on_gpu():
    w = make_workload(Spec("agree", 2, 2, 128, 1024, 8192, values="spread"), seed=5)
    o1, l1, _ = _decode(w, num_parts=4)            # one part per row
    o2, l2, md = _decode(w, num_parts=13)          # rows split
    assert md.workspace is not None
    ref_out, ref_lse = _oracle(w)
    check_rows(o1, l1, ref_out, ref_lse, "unsplit")
    check_rows(o2, l2, ref_out, ref_lse, "split")


def test_combine_matches_oracle_merge():
    spec = Spec("comb", 3, 1, 32, 600, 4096, neg="tail10")
    w = make_workload(spec, seed=3)
    sched, split_ptr, _ = oracle_metadata(3, 1, 600, 0, 7, 1)
    po, pl = oracle_split_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"], sched,
                                 split_ptr)
    po32, pl32 = po.astype(np.float32), pl.astype(np.float32)
    ref_out, ref_lse = oracle_combine(po32.astype(np.float64), pl32.astype(np.float64), split_ptr)
    out, lse = mla.combine(torch.from_numpy(po32).cuda(), torch.from_numpy(pl32).cuda(),
                           torch.from_numpy(split_ptr).cuda())
    torch.cuda.synchronize()
    check_rows(out, lse, ref_out, ref_lse, "combine")


def test_combine_many_splits_across_batches():
    # rows of 1, 9, 20 and 17 splits: the merge takes splits eight at a time, so the running maximum
    # rises between batches; row 3's first batch is all empty, and its lse spread is wide
    rng = np.random.default_rng(11)
    counts = [1, 9, 20, 17]
    split_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    s, h = int(split_ptr[-1]), 8
    po = rng.standard_normal((s, h, 512)).astype(np.float32)
    pl = rng.uniform(-30.0, 30.0, (s, h)).astype(np.float32)
    pl[split_ptr[2] + 3] = -np.inf                   # a dead split inside a batch
    pl[split_ptr[3]:split_ptr[3] + 8] = -np.inf      # row 3: its first batch has no live split
    pl[split_ptr[3] + 12, :4] = 80.0                 # a later batch raises the maximum a lot
    ref_out, ref_lse = oracle_combine(po.astype(np.float64), pl.astype(np.float64), split_ptr)
    out, lse = mla.combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                           torch.from_numpy(split_ptr).cuda())
    torch.cuda.synchronize()
    check_rows(out, lse, ref_out, ref_lse, "combine, many splits")


def test_combine_all_empty_splits():
    po = torch.zeros((3, 4, 512), device="cuda")
    pl = torch.full((3, 4), -math.inf, device="cuda")
    sp = torch.tensor([0, 2, 3], dtype=torch.int32, device="cuda")
    out, lse = mla.combine(po, pl, sp)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_validate_indices_counts_out_of_pool_entries():
    idx = torch.tensor([0, 5, -1, 9, 10, 11, -7, 3], dtype=torch.int32, device="cuda")
    assert mla.validate_indices(idx, 10) == 2
    assert mla.validate_indices(idx, 100) == 0


# ----------------------------------------------------------- full-size workloads, every row checked

@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_full_size_workloads_every_row(cfg):
    """The five workloads at full size, in the launch configuration the benchmark times (default
    schedule), every query row compared with the oracle."""
    w = make_workload(cfg)
    out, lse, md = _decode(w)
    spec = w["spec"]
    nrows = spec.rows
    print(f"config {cfg}: {nrows} rows, {md.num_parts} parts", flush=True)
    o = out.reshape(nrows, spec.h_q, 512)
    l = lse.reshape(nrows, spec.h_q)
    step = 32
    for r0 in range(0, nrows, step):
        rows = list(range(r0, min(nrows, r0 + step)))
        ref_out, ref_lse = oracle_decode_rows(w["q_bits"], w["k_cache"], w["indices"],
                                              w["softmax_scale"], rows, w["extra_k_cache"],
                                              w["extra_indices"])
        check_rows(o[rows], l[rows], ref_out, ref_lse, f"config {cfg} rows {rows[0]}..{rows[-1]}")


def test_check_indices_reports_out_of_pool_entries():
    idx = torch.tensor([0, 5, -1, 9, -7, 3], dtype=torch.int32, device="cuda")
    assert mla.check_indices(idx, 10) is True
    assert mla.check_indices(idx, 9) is False
    assert mla.check_indices(idx[:0], 1) is True


@pytest.mark.parametrize("h_q,extra", [(128, 0), (64, 0), (64, 40)])
def test_duplicate_entries_count_with_multiplicity(h_q, extra):
    """Every selected token listed twice (the row's second half repeats its first half), and one row
    that lists a single token 300 times: the softmax runs over the list as given, so the output is
    that of the distinct tokens and lse grows by ln 2 (resp. equals s + ln 300)."""
    spec = Spec("dups", 2, 1, h_q, 300, 2048, extra_topk=extra,
                extra_tokens_per_seq=1024 if extra else 0)
    w = make_workload(spec, seed=41)
    base_out, base_lse = _oracle(w)
    idx = w["indices"]
    idx[:, :, 150:] = idx[:, :, :150]                    # every entry twice
    idx[1, 0, :] = idx[1, 0, 7]                          # row 1: one token, 300 times
    if extra:
        w["extra_indices"][:, :, 20:] = w["extra_indices"][:, :, :20]
    ref_out, ref_lse = _oracle(w)
    out, lse, _ = _decode(w)
    check_rows(out, lse, ref_out, ref_lse, f"dups/h{h_q}")
    assert np.isfinite(ref_lse).all()
    # the oracle's own reading of duplicates, for the doubled row 0
    if not extra:
        half = dict(w)
        half["indices"] = idx[:, :, :150].copy()
        h_out, h_lse = _oracle(half)
        assert np.allclose(ref_lse[0], h_lse[0] + math.log(2.0), atol=1e-9)


@pytest.mark.parametrize("h_q", [128, 64])
def test_decode_replays_from_a_captured_graph(h_q):
    """The decode step captured in a HIP graph (through torch.cuda.CUDAGraph): every replay, with
    eager work on the same stream between replays, matches the eager result bit for bit. Both
    kernels (128-head groups with fp32 partials, 64-head groups with bf16 partials) and their
    merges are captured."""
    spec = Spec("graph", 4, 2, h_q, 700, 4096, neg="tail10")
    w = make_workload(spec, seed=51)
    d = to_dev(w)
    md = mla.get_metadata(4, 2, h_q, 700, 0, num_parts=13)      # rows split: decode + merge
    assert md.workspace is not None
    out = torch.empty((4, 2, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((4, 2, h_q), dtype=torch.float32, device="cuda")
    mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md, out=out, lse=lse)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md,
                              out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(k + 1.0)                                  # eager work between the replays
        lse.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {k}: output differs from the eager decode"
        assert torch.equal(lse, eager_lse), f"replay {k}: lse differs from the eager decode"
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, "graph")


# ------------------------------------------------ the single-stream 64-head kernel (mla_decode_h64)
# h_q <= 64 runs in that kernel when the parts average at least 6 sub-tiles of 32 tokens
# (2 * rows * units / parts >= 6), or 8 with an extra cache (units of both caches), as the default
# schedules of the larger shapes do; the cases below are sized for it. Parts of fewer sub-tiles run
# the two-half kernel (mla_decode.hip).

def _stream_parts(spec, per_part):
    """A part count that gives `per_part` sub-tiles per part (at least 6, or 8 with an extra cache),
    units of both caches."""
    units = -(-spec.topk // 64) + -(-spec.extra_topk // 64)
    parts = max(1, 2 * spec.rows * units // per_part)
    assert 2 * spec.rows * units >= (8 if spec.extra_topk else 6) * parts
    return parts


@pytest.mark.parametrize("spec,per_part", [
    (Spec("stream_h64_whole_rows", 2, 2, 64, 1024, 4096, neg="tail10"), 32),
    (Spec("stream_h64_split", 2, 2, 64, 1024, 4096, values="spread"), 16),
    (Spec("stream_h40_multi_segment", 3, 2, 40, 700, 4096, neg="frac5"), 14),
    (Spec("stream_h16", 2, 1, 16, 2048, 8192), 64),
    (Spec("stream_h16_split", 2, 1, 16, 2048, 8192, neg="tail10"), 24),
    (Spec("stream_h64_ragged_topk", 1, 3, 64, 1000, 8192, neg="frac5"), 32),
], ids=lambda x: x.name if isinstance(x, Spec) else str(x))
def test_decode_single_stream_64_head_kernel(spec, per_part):
    w = make_workload(spec, seed=41)
    out, lse, md = _decode(w, num_parts=_stream_parts(spec, per_part))
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, spec.name)


@pytest.mark.parametrize("per_part", [32, 16])
def test_stream_64_head_trailing_ignored_subtiles(per_part):
    """As test_decode_trailing_ignored_subtiles, for the single-stream 64-head kernel: rows whose
    selections end in runs of -1 of every length relative to the sub-tile, a fully ignored sub-tile
    inside the live part, whole rows with no valid entry."""
    spec = Spec("trailing64", 4, 2, 64, 1024, 4096)
    w = make_workload(spec, seed=33)
    idx = w["indices"].reshape(8, 1024)
    for r, n_live in enumerate([0, 1, 31, 32, 33, 95, 500, 1024]):
        idx[r, n_live:] = -1
    idx[6, 64:96] = -1
    idx[7, 1023] = -1
    out, lse, md = _decode(w, num_parts=_stream_parts(spec, per_part))
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, f"trailing64/{per_part}")
    assert torch.all(lse[0, 0] == -math.inf)
    assert torch.all(out[0, 0] == 0)


@pytest.mark.parametrize("spec,per_part", [
    # parts cut rows inside either cache's sub-tiles and across the boundary between them
    (Spec("long_parts_mixed_split", 2, 2, 64, 1000, 4096, extra_topk=300, extra_tokens_per_seq=2048,
          neg="frac5"), 14),
    (Spec("long_parts_mixed_whole_rows", 2, 1, 64, 2048, 8192, extra_topk=512,
          extra_tokens_per_seq=2048), 80),
    # fp8 list ending 13 tokens into its last unit, so its last sub-tile is empty before the
    # fp4 sub-tiles start
    (Spec("long_parts_h16_mixed_ragged", 1, 3, 16, 333, 4096, extra_topk=129, extra_tokens_per_seq=1024,
          values="spread"), 12),
    (Spec("long_parts_fp4_only", 2, 2, 64, 0, 64, extra_topk=800, extra_tokens_per_seq=4096,
          neg="tail10"), 13),
    (Spec("long_parts_h40_mixed", 3, 1, 40, 700, 4096, extra_topk=200, extra_tokens_per_seq=1024), 16),
], ids=lambda x: x.name if isinstance(x, Spec) else str(x))
def test_decode_64_head_extra_cache_long_parts(spec, per_part):
    """Extra-cache decodes in the single-stream kernel (parts of 12 and more sub-tiles), whose
    segments start inside either cache's sub-tiles or cross from the one to the other."""
    w = make_workload(spec, seed=43)
    out, lse, md = _decode(w, num_parts=_stream_parts(spec, per_part))
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, spec.name)


@pytest.mark.parametrize("per_part", [24, 12])
def test_64_head_ignored_runs_in_either_cache(per_part):
    """Extra-cache decodes with rows that have no valid entry in either list, in only one of them,
    and runs of -1 ending each list part-way through a sub-tile."""
    spec = Spec("ignored_mixed", 5, 1, 64, 512, 4096, extra_topk=256, extra_tokens_per_seq=1024)
    w = make_workload(spec, seed=37)
    idx = w["indices"].reshape(5, 512)
    xidx = w["extra_indices"].reshape(5, 256)
    idx[0] = -1
    xidx[0] = -1
    idx[1] = -1
    xidx[2] = -1
    idx[3, 100:] = -1
    xidx[3, 33:] = -1
    idx[4, 200:480] = -1
    xidx[4, :64] = -1
    out, lse, md = _decode(w, num_parts=_stream_parts(spec, per_part))
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, f"ignored_mixed/{per_part}")
    assert torch.all(lse[0, 0] == -math.inf)
    assert torch.all(out[0, 0] == 0)


@pytest.mark.parametrize("spec,per_part", [
    (Spec("two_half_h64", 2, 2, 64, 1000, 4096, neg="frac5"), 4),
    (Spec("two_half_h64_spread", 2, 1, 64, 2048, 8192, values="spread", neg="tail10"), 2),
    (Spec("two_half_h16", 3, 1, 16, 700, 4096), 4),
    (Spec("two_half_h40_multi_segment", 3, 2, 40, 333, 2048, neg="frac5"), 3),
    (Spec("two_half_h64_mixed", 2, 2, 64, 500, 4096, extra_topk=200, extra_tokens_per_seq=1024,
          neg="frac5"), 4),
    (Spec("two_half_h32_fp4_only", 3, 1, 32, 0, 64, extra_topk=300, extra_tokens_per_seq=1024), 2),
], ids=lambda x: x.name if isinstance(x, Spec) else str(x))
def test_decode_two_half_kernel_short_parts(spec, per_part):
    """Decodes whose parts average fewer than 6 sub-tiles, which run the two-half 64-head kernel
    (mla_decode.hip) rather than the single-stream one."""
    units = -(-spec.topk // 64) + -(-spec.extra_topk // 64)
    parts = -(-2 * spec.rows * units // per_part)
    assert 2 * spec.rows * units < 6 * parts
    w = make_workload(spec, seed=47)
    out, lse, md = _decode(w, num_parts=parts)
    ref_out, ref_lse = _oracle(w)
    check_rows(out, lse, ref_out, ref_lse, spec.name)


def test_stream_64_head_full_size_mid_workload():
    """The mid workload (batch 32, h_q 64, topk 2048) at 64 parts, which runs the single-stream
    kernel with two parts per row: every row against the oracle."""
    w = make_workload(1)
    spec = w["spec"]
    out, lse, md = _decode(w, num_parts=64)
    assert md.workspace is not None
    o = out.reshape(spec.rows, spec.h_q, 512)
    l = lse.reshape(spec.rows, spec.h_q)
    for r0 in range(0, spec.rows, 16):
        rows = list(range(r0, min(spec.rows, r0 + 16)))
        ref_out, ref_lse = oracle_decode_rows(w["q_bits"], w["k_cache"], w["indices"],
                                              w["softmax_scale"], rows)
        check_rows(o[rows], l[rows], ref_out, ref_lse, f"mid/64 parts rows {rows[0]}..{rows[-1]}")
