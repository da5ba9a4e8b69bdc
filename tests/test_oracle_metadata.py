"""Pins for the oracle's tile-scheduler metadata (CPU only): hand-derived fixtures and invariants."""
import itertools
import os

import numpy as np
import pytest

from oracle import oracle_metadata, part_count, tiles_per_row


def _cases(golden_dir):
    cases, cur = [], None
    for ln in open(os.path.join(golden_dir, "metadata_small.txt")):
        ln = ln.split("#")[0].strip()
        if not ln:
            continue
        tok = ln.split()
        if tok[0] == "case":
            cur = dict(name=tok[1], args=[int(x) for x in tok[2:]], sched={})
            cases.append(cur)
        elif tok[0] == "parts":
            cur["parts"] = int(tok[1])
        elif tok[0] == "split_ptr":
            cur["split_ptr"] = [int(x) for x in tok[1:]]
        elif tok[0] == "sched":
            cur["sched"][int(tok[1])] = [int(x) for x in tok[2:]]
    return cases


def test_hand_derived_cases(golden_dir):
    cases = _cases(golden_dir)
    assert len(cases) == 4
    for c in cases:
        b, s, topk, extra, parts, min_tiles = c["args"]
        sched, split_ptr, p_eff = oracle_metadata(b, s, topk, extra, parts, min_tiles)
        assert p_eff == c["parts"], c["name"]
        assert list(split_ptr) == c["split_ptr"], c["name"]
        for p, fields in c["sched"].items():
            assert list(sched[p, :5]) == fields, (c["name"], p)
            assert list(sched[p, 5:]) == [0, 0, 0]


def test_tiles_per_row():
    assert tiles_per_row(128, 0) == 2 and tiles_per_row(2048, 512) == 40
    assert tiles_per_row(1, 0) == 1 and tiles_per_row(0, 0) == 1 and tiles_per_row(65, 1) == 3
    assert tiles_per_row(131072, 0) == 2048


@pytest.mark.parametrize("batch,seq,topk,extra,parts,min_tiles", list(itertools.product(
    [1, 3, 8], [1, 2], [1, 64, 100, 2048], [0, 70], [1, 5, 64, 256], [1, 4])))
def test_partition_invariants(batch, seq, topk, extra, parts, min_tiles):
    rows = batch * seq
    tiles = tiles_per_row(topk, extra)
    units = rows * tiles
    sched, split_ptr, p_eff = oracle_metadata(batch, seq, topk, extra, parts, min_tiles)
    assert p_eff == part_count(rows, tiles, parts, min_tiles)
    assert 1 <= p_eff <= parts and (units < min_tiles or p_eff <= units // min_tiles)
    starts = sched[:, 0].astype(np.int64) * tiles + sched[:, 1]
    ends = sched[:, 2].astype(np.int64) * tiles + sched[:, 3]
    # contiguous, ordered, covering every unit exactly once
    assert starts[0] == 0 and ends[-1] == units
    assert np.all(starts[1:] == ends[:-1]) and np.all(ends >= starts)
    sizes = ends - starts
    assert sizes.max() - sizes.min() <= 1
    assert np.all(sched[:, 1] < tiles) and np.all(sched[:, 3] < tiles)
    # splits per row = parts meeting that row, slots in part order
    meets = [[p for p in range(p_eff) if starts[p] < (r + 1) * tiles and ends[p] > r * tiles]
             for r in range(rows)]
    assert list(np.diff(split_ptr)) == [len(m) for m in meets]
    assert split_ptr[0] == 0 and split_ptr[-1] <= rows + p_eff - 1
    for p in range(p_eff):
        if sizes[p]:
            r0 = int(starts[p] // tiles)
            assert sched[p, 4] == split_ptr[r0] + meets[r0].index(p)


def test_depends_only_on_integers():
    a = oracle_metadata(4, 2, 300, 10, 13, 2)
    b = oracle_metadata(4, 2, 300, 10, 13, 2)
    assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2])) and a[2] == b[2]


def test_headline_shape_is_one_split_per_row():
    sched, split_ptr, p_eff = oracle_metadata(128, 2, 2048, 0, 256, 1)
    assert p_eff == 256 and np.all(np.diff(split_ptr) == 1)
    assert np.all(sched[:, 1] == 0) and np.all(sched[:, 0] == np.arange(256))
