"""Tile-scheduler metadata: the partition of (row, tile) work units over parts, in plain Python.

Test infrastructure (see the package docstring): never used by the product path.

The pages state only that the tile-scheduler metadata is computed once, before the decode loop, and
that decoding is split with num_splits (page "flops/flashmla-decode-fp8-fp4-kv", section
"Workarounds"; page "deepseek-ai/FlashMLA", section "How to use it": first obtain the scheduler
metadata, then call the decode for every generation step). Its content is therefore this project's
own specification, stated here and reproduced bit-for-bit by the device kernel:

* A query row r = b * seq_len_q + s owns ``tiles`` units of TILE_TOKENS (=64) token slots:
  ceil(topk / 64) units over the fp8 index list, then ceil(extra_topk / 64) over the fp4 one (a unit
  never mixes the two caches); a row always owns at least one unit.
* Units are numbered u = r * tiles + t, U = rows * tiles in all.
* P_eff = max(1, min(num_parts, U // min_tiles_per_part)) parts; part p covers the contiguous units
  [floor(p * U / P_eff), floor((p + 1) * U / P_eff)), so part sizes differ by at most one unit.
* num_splits[r] = the number of parts whose range meets row r; split_ptr is its exclusive prefix sum
  (length rows + 1). The splits of row r occupy workspace slots split_ptr[r] .. split_ptr[r+1]-1 in
  part order.
* sched[p] = (begin_row, begin_tile, end_row, end_tile, first_slot, 0, 0, 0) where (end_row,
  end_tile) is the exclusive end unit (end_tile may be 0 of the next row) and first_slot is the slot
  of part p's split of its first row.

Nothing depends on the index values: the metadata is a pure function of these integers.
"""
import numpy as np

TILE_TOKENS = 64
SCHED_FIELDS = 8


def tiles_per_row(topk: int, extra_topk: int) -> int:
    """Units per row: fp8 units, then fp4 units; at least one."""
    t = -(-topk // TILE_TOKENS) + -(-extra_topk // TILE_TOKENS)
    return max(1, t)


def part_count(rows: int, tiles: int, num_parts: int, min_tiles_per_part: int) -> int:
    """P_eff = max(1, min(num_parts, U // min_tiles_per_part)) with U = rows * tiles."""
    units = rows * tiles
    return max(1, min(num_parts, units // min_tiles_per_part))


def oracle_metadata(batch: int, seq_len_q: int, topk: int, extra_topk: int, num_parts: int,
                    min_tiles_per_part: int = 1):
    """Return (sched int32 [P_eff, 8], split_ptr int32 [rows + 1], P_eff) following the spec above.

    Written the slow way: every unit is walked and assigned to its part by the range definition.
    """
    if num_parts < 1 or min_tiles_per_part < 1:
        raise ValueError("num_parts and min_tiles_per_part must be >= 1")
    rows = batch * seq_len_q
    tiles = tiles_per_row(topk, extra_topk)
    units = rows * tiles
    parts = part_count(rows, tiles, num_parts, min_tiles_per_part)
    begin = [(p * units) // parts for p in range(parts)]
    end = [((p + 1) * units) // parts for p in range(parts)]

    # which parts meet each row, in part order
    parts_of_row = [[] for _ in range(rows)]
    for p in range(parts):
        for u in range(begin[p], end[p]):
            r = u // tiles
            if not parts_of_row[r] or parts_of_row[r][-1] != p:
                parts_of_row[r].append(p)

    split_ptr = np.zeros(rows + 1, dtype=np.int32)
    for r in range(rows):
        split_ptr[r + 1] = split_ptr[r] + len(parts_of_row[r])

    sched = np.zeros((parts, SCHED_FIELDS), dtype=np.int32)
    for p in range(parts):
        b, e = begin[p], end[p]
        sched[p, 0], sched[p, 1] = divmod(b, tiles)
        sched[p, 2], sched[p, 3] = divmod(e, tiles)
        if b < e:
            r0 = b // tiles
            sched[p, 4] = split_ptr[r0] + parts_of_row[r0].index(p)
        else:                                   # empty part (only when units == 0)
            sched[p, 4] = split_ptr[min(b // tiles, rows)] if rows else 0
    return sched, split_ptr, parts
