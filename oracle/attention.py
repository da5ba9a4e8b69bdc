"""Sparse MLA decode attention, its split form and the log-sum-exp merge, in float64.

Test infrastructure (see the package docstring): never used by the product path.

What is computed (the plain definition; the method reaches the same result faster):

* MLA decode in absorbed form reads one latent head per token, shared by every query head, and the
  value is that same 512-dim latent (page "flops/flashmla-decode-fp8-fp4-kv", section "Arithmetic
  intensity"; page "flops/attn-mla-kernel-support-matrix", section "Workarounds", MLA absorbed form).
* An indices tensor of shape (batch, seq_len_q, topk) selects each query row's tokens; -1 entries are
  ignored and unselected KV is never touched (page "flops/flashmla-decode-fp8-fp4-kv", section
  "Workarounds"; page "deepseek-ai/FlashMLA", section "Key technical details"). Every negative entry
  is read as "ignored"; an entry at or past the pool size is a precondition violation (ValueError).
* An optional fp4 extra cache (valid only next to an fp8 k_cache, same page, "Arithmetic intensity")
  is selected by its own (batch, seq_len_q, extra_topk) indices; the row attends with one softmax
  over the union of both selections, counted with multiplicity.
* The decode returns the output and the natural-log log-sum-exp of the scores (page
  "deepseek-ai/FlashMLA", section "How to use it"). For head h of a row with selected latents
  k_1..k_n: s_t = scale * <q_h, k_t>, lse = log(sum_t exp(s_t)), out = sum_t exp(s_t - lse) k_t.
  A row with no valid entry has out = 0 and lse = -inf.
* Split decoding with num_splits (page "flops/flashmla-decode-fp8-fp4-kv", section "Workarounds"):
  each split attends over its own share of a row's tokens and yields (o_i, lse_i) with o_i already
  normalised; the merge is M = max_i lse_i, w_i = exp(lse_i - M), lse = M + log(sum w_i),
  out = sum_i w_i o_i / sum_i w_i, which equals the unsplit result exactly in exact arithmetic.
"""
import numpy as np

from .formats import HEAD_DIM, bf16_bits_to_f64, dequant_fp4_records, dequant_fp8_records
from .metadata import TILE_TOKENS, tiles_per_row


def _as_q(q):
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return bf16_bits_to_f64(q)
    return q.astype(np.float64)


def _check_range(sel: np.ndarray, n_tokens: int, what: str):
    if sel.size and int(sel.max()) >= n_tokens:
        raise ValueError(f"{what} index {int(sel.max())} is outside the pool of {n_tokens} tokens")


def _attend(q_row: np.ndarray, latents: np.ndarray, softmax_scale: float):
    """q_row [H, 512], latents [n, 512] -> (out [H, 512], lse [H]) by the plain definition."""
    h = q_row.shape[0]
    if latents.shape[0] == 0:
        return np.zeros((h, HEAD_DIM)), np.full(h, -np.inf)
    s = softmax_scale * (q_row @ latents.T)                         # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    out = np.exp(s - lse[:, None]) @ latents
    return out, lse


def row_token_lists(indices_row, extra_indices_row=None):
    """The valid entries of one row's index lists (negative entries dropped, order kept)."""
    sel = np.asarray(indices_row).reshape(-1)
    sel = sel[sel >= 0]
    sel_x = None
    if extra_indices_row is not None:
        sel_x = np.asarray(extra_indices_row).reshape(-1)
        sel_x = sel_x[sel_x >= 0]
    return sel, sel_x


def _gather(k_cache, extra_k_cache, sel, sel_x):
    k8 = np.asarray(k_cache, dtype=np.uint8).reshape(-1, 528)
    _check_range(sel, k8.shape[0], "k_cache")
    parts = [dequant_fp8_records(k8[sel])]
    if sel_x is not None and extra_k_cache is not None:
        k4 = np.asarray(extra_k_cache, dtype=np.uint8).reshape(-1, 288)
        _check_range(sel_x, k4.shape[0], "extra_k_cache")
        parts.append(dequant_fp4_records(k4[sel_x]))
    return np.concatenate(parts, axis=0)


def oracle_decode_rows(q, k_cache, indices, softmax_scale, rows, extra_k_cache=None,
                       extra_indices=None):
    """Decode only the listed flat rows r = b * seq_len_q + s. Returns (out [len, H, 512], lse [len, H])."""
    qf = _as_q(q)
    b_, s_, h_, d_ = qf.shape
    assert d_ == HEAD_DIM
    idx = np.asarray(indices).reshape(b_ * s_, -1)
    xidx = None if extra_indices is None else np.asarray(extra_indices).reshape(b_ * s_, -1)
    qr = qf.reshape(b_ * s_, h_, d_)
    outs, lses = [], []
    for r in rows:
        sel, sel_x = row_token_lists(idx[r], None if xidx is None else xidx[r])
        lat = _gather(k_cache, extra_k_cache, sel, sel_x)
        o, l = _attend(qr[r], lat, softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def oracle_decode(q, k_cache, indices, softmax_scale, extra_k_cache=None, extra_indices=None):
    """Full decode. q: bf16 bits (uint16) or floats [B, S, H, 512]; k_cache uint8 [..., 528];
    indices int [B, S, topk]; optional extra_k_cache uint8 [..., 288] and extra_indices [B, S, extra].
    Returns out float64 [B, S, H, 512] and lse float64 [B, S, H]."""
    qf = _as_q(q)
    b_, s_, h_, _ = qf.shape
    out, lse = oracle_decode_rows(qf, k_cache, indices, softmax_scale, range(b_ * s_),
                                  extra_k_cache, extra_indices)
    return out.reshape(b_, s_, h_, HEAD_DIM), lse.reshape(b_, s_, h_)


def _unit_tokens(idx_row, xidx_row, topk, extra_topk, tile):
    """Index entries of one 64-slot unit: fp8 units first, then fp4 units."""
    tiles_k = -(-topk // TILE_TOKENS)
    if tile < tiles_k:
        return idx_row[tile * TILE_TOKENS: min((tile + 1) * TILE_TOKENS, topk)], None
    t = tile - tiles_k
    return None, xidx_row[t * TILE_TOKENS: min((t + 1) * TILE_TOKENS, extra_topk)]


def oracle_split_decode(q, k_cache, indices, softmax_scale, sched, split_ptr, extra_k_cache=None,
                        extra_indices=None):
    """Per-split partial results following the metadata partition.

    Returns (partial_o [S_total, H, 512], partial_lse [S_total, H]); slot split_ptr[r] + i holds the
    i-th split of row r (parts in order), o normalised by its own softmax sum.
    """
    qf = _as_q(q)
    b_, s_, h_, d_ = qf.shape
    rows = b_ * s_
    idx = np.asarray(indices).reshape(rows, -1)
    topk = idx.shape[1]
    xidx = None if extra_indices is None else np.asarray(extra_indices).reshape(rows, -1)
    extra_topk = 0 if xidx is None else xidx.shape[1]
    tiles = tiles_per_row(topk, extra_topk)
    qr = qf.reshape(rows, h_, d_)
    total = int(split_ptr[-1])
    po = np.zeros((total, h_, d_))
    pl = np.full((total, h_), -np.inf)
    for p in range(sched.shape[0]):
        u0 = int(sched[p, 0]) * tiles + int(sched[p, 1])
        u1 = int(sched[p, 2]) * tiles + int(sched[p, 3])
        u = u0
        while u < u1:
            r = u // tiles
            seg_end = min(u1, (r + 1) * tiles)
            slot = int(sched[p, 4]) if u == u0 else int(split_ptr[r])
            sel_parts, selx_parts = [], []
            for t in range(u - r * tiles, seg_end - r * tiles):
                a, bx = _unit_tokens(idx[r], None if xidx is None else xidx[r], topk, extra_topk, t)
                if a is not None:
                    sel_parts.append(a)
                if bx is not None:
                    selx_parts.append(bx)
            sel = np.concatenate(sel_parts) if sel_parts else np.zeros(0, dtype=np.int64)
            sel = sel[sel >= 0]
            sel_x = None
            if selx_parts:
                sel_x = np.concatenate(selx_parts)
                sel_x = sel_x[sel_x >= 0]
            lat = _gather(k_cache, extra_k_cache, sel, sel_x)
            po[slot], pl[slot] = _attend(qr[r], lat, softmax_scale)
            u = seg_end
    return po, pl


def oracle_combine(partial_o, partial_lse, split_ptr):
    """Log-sum-exp merge of each row's splits. Returns (out [rows, H, 512], lse [rows, H]).

    A row whose splits all have lse = -inf (no valid token anywhere) gets out = 0, lse = -inf.
    """
    partial_o = np.asarray(partial_o, dtype=np.float64)
    partial_lse = np.asarray(partial_lse, dtype=np.float64)
    rows = len(split_ptr) - 1
    h_, d_ = partial_o.shape[1], partial_o.shape[2]
    out = np.zeros((rows, h_, d_))
    lse = np.full((rows, h_), -np.inf)
    for r in range(rows):
        a, b = int(split_ptr[r]), int(split_ptr[r + 1])
        if b <= a:
            continue
        lses = partial_lse[a:b]                                      # [n, H]
        m = lses.max(axis=0)                                         # [H]
        live = np.isfinite(m)
        msafe = np.where(live, m, 0.0)
        w = np.where(np.isfinite(lses), np.exp(lses - msafe[None, :]), 0.0)   # [n, H]
        wsum = w.sum(axis=0)
        lse[r] = np.where(live, msafe + np.log(np.where(live, wsum, 1.0)), -np.inf)
        num = (w[:, :, None] * partial_o[a:b]).sum(axis=0)
        out[r] = np.where(live[:, None], num / np.where(live, wsum, 1.0)[:, None], 0.0)
    return out, lse
