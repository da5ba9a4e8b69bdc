"""GPU parity of the fused decode (mla_sparse_decode_fused) with oracle/fused.py.

Two roundings decide discrete values from floating point, and the kernel takes them from fp32
values that differ slightly from the oracle's exact ones:

* the normalised, rotated query is rounded to bf16: where the exact value lies within the kernel's
  fp32 error bound of a bf16 tie (2^-21 relative for the normalised dims; 2^-20 (|x0| + |x1|) for a
  rotated pair), the kernel may round the other way. For each (row, head) the test adds to the
  tolerances the largest score change such flips can cause, B = scale * sum over those elements of
  one bf16 step times the largest |key| in that dim: lse within 1e-3 + B, and the output within
  2 B * max|V| more. Heads without such an element (nearly all) keep the plain decode's bar;
* the output is cast to fp8: a value next to an e4m3 rounding boundary may land on the neighbouring
  code, so each dequantized output value must lie within the decode tolerance (2e-2 * max|ref| of
  its row) plus half an e4m3 step at the kernel's block scale of the oracle's exact pre-cast value;
  scale bytes within one of the oracle's, and at least 90% of the record bytes identical to the
  oracle's."""
import math

import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import (E4M3, E8M0, bf16_bits_to_f64, dequant_fp4_records, dequant_fp8_records,
                    row_token_lists)
from oracle.fused import oracle_fused_decode, rms_norm, rope
from workloads import Spec, make_workload
from tests.gpu_helpers import LSE_ABS_TOL, OUT_REL_TOL, to_dev

pytestmark = pytest.mark.gpu


def _rope_tables(rows, seed):
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, 65536, rows).astype(np.float64)
    inv_freq = 10000.0 ** (-np.arange(32) / 32.0)
    ang = pos[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _dequant(rec):
    data = E4M3[rec[..., :512]]
    sc = E8M0[rec[..., 512:]]
    return data * np.repeat(sc, 32, axis=-1)


def _flip_bounds(w, wbits, eps, cos, sin):
    """Per (row, head): B (largest score change from query elements whose bf16 rounding the kernel
    may take the other way) and the row's largest |V| value."""
    spec = w["spec"]
    rows, h = spec.rows, spec.h_q
    q = bf16_bits_to_f64(w["q_bits"]).reshape(rows, h, 512)
    x = rms_norm(q, bf16_bits_to_f64(wbits), eps)
    c = cos.reshape(rows, 1, 32).astype(np.float64)
    sn = sin.reshape(rows, 1, 32).astype(np.float64)
    pre = rope(x, c, sn)
    err = 2.0 ** -21 * np.abs(pre)
    pair = np.abs(x[..., 448::2]) + np.abs(x[..., 449::2])
    err[..., 448::2] = 2.0 ** -20 * pair
    err[..., 449::2] = 2.0 ** -20 * pair
    mag = np.abs(pre)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    step = np.exp2(np.maximum(e, -126) - 7)
    tie = (np.floor(pre / step) + 0.5) * step
    near = (np.abs(pre - tie) <= err) & (mag > 0)
    idx = w["indices"].reshape(rows, -1)
    xidx = None if w["extra_indices"] is None else w["extra_indices"].reshape(rows, -1)
    bound = np.zeros((rows, h))
    vmax = np.zeros(rows)
    for r in range(rows):
        sel, sel_x = row_token_lists(idx[r], None if xidx is None else xidx[r])
        lat = [dequant_fp8_records(w["k_cache"][sel])]
        if sel_x is not None and sel_x.size:
            lat.append(dequant_fp4_records(w["extra_k_cache"][sel_x]))
        lat = np.concatenate(lat)
        if lat.shape[0] == 0:
            continue
        kmax = np.abs(lat).max(axis=0)                                # [512]
        vmax[r] = kmax.max()
        bound[r] = spec.softmax_scale * (near[r] * step[r] * kmax[None, :]).sum(axis=1)
    return bound, vmax


def _check(rec_gpu, lse_gpu, rec_ref, lse_ref, out_ref, what, bound, vmax):
    rows = rec_ref.reshape(-1, rec_ref.shape[-2], 528).shape[0]
    g = rec_gpu.reshape(rows, -1, 528)
    r = rec_ref.reshape(rows, -1, 528)
    o = out_ref.reshape(rows, -1, 512)
    lg, lr = lse_gpu.reshape(rows, -1), lse_ref.reshape(rows, -1)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: -inf pattern"
    fin = ~np.isneginf(lr)
    if fin.any():
        d = np.abs(lg - lr)[fin] - bound[fin]
        assert d.max() <= LSE_ABS_TOL, f"{what}: |d lse| - B = {d.max():.3e}"
    assert np.abs(g[..., 512:].astype(int) - r[..., 512:].astype(int)).max() <= 1, f"{what}: scale bytes"
    deq = _dequant(g)
    k = E8M0[g[..., 512:]]                                            # block scales (powers of two)
    y = np.abs(deq) / np.repeat(k, 32, axis=-1)                       # the e4m3 values
    step = np.where(y >= 2 ** -6, np.exp2(np.floor(np.log2(np.maximum(y, 2 ** -6))) - 3), 2 ** -9)
    half = 0.5 * step * np.repeat(k, 32, axis=-1)
    for i in range(rows):
        tol = OUT_REL_TOL * np.abs(o[i]).max() + half[i] + 2 * bound[i][:, None] * vmax[i]
        bad = np.abs(deq[i] - o[i]) > tol
        assert not bad.any(), f"{what}: row {i}, {bad.sum()} values off"
    # codes next to a rounding boundary may differ (a few percent of the bytes, from the decode's
    # own ~1e-3 relative error against e4m3 steps of 2^-4); a wrong scale rule, rounding mode or
    # byte order would leave far fewer bytes identical
    same = (g == r).mean()
    assert same >= 0.9, f"{what}: only {same:.3f} of the record bytes match the oracle's"


CASES = [
    (Spec("fz_h128", 2, 2, 128, 700, 8192, values="spread", neg="tail10"), 0),
    (Spec("fz_h128_split", 3, 1, 128, 1500, 8192, neg="frac5"), 17),
    (Spec("fz_h128_mixed", 2, 1, 128, 300, 4096, extra_topk=100, extra_tokens_per_seq=2048), 0),
    (Spec("fz_h200", 1, 2, 200, 300, 4096, neg="frac5"), 5),
    (Spec("fz_h128_empty", 2, 1, 128, 80, 1024, neg="all"), 0),
]


@pytest.mark.parametrize("spec,parts", CASES, ids=[c[0].name for c in CASES])
def test_fused_decode_matches_oracle(spec, parts):
    w = make_workload(spec, seed=81)
    rows = spec.rows
    rng = np.random.default_rng(82)
    wt = torch.from_numpy((1 + 0.1 * rng.standard_normal(512)).astype(np.float32)).to(torch.bfloat16)
    cos, sin = _rope_tables(rows, 83)
    eps = 1e-6
    d = to_dev(w)
    md = mla.get_metadata(spec.batch, spec.seq_len_q, spec.h_q, spec.topk, spec.extra_topk,
                          num_parts=parts)
    if parts:
        assert md.workspace is not None
    c3 = torch.from_numpy(cos.reshape(spec.batch, spec.seq_len_q, 32)).cuda()
    s3 = torch.from_numpy(sin.reshape(spec.batch, spec.seq_len_q, 32)).cuda()
    rec, lse = mla.sparse_decode_fused(d["q"], wt.cuda(), eps, c3, s3, d["k_cache"], d["indices"],
                                       w["softmax_scale"], md, d.get("extra_k_cache"),
                                       d.get("extra_indices"))
    torch.cuda.synchronize()
    wbits = wt.view(torch.int16).numpy().view(np.uint16)
    rec_ref, lse_ref, out_ref = oracle_fused_decode(
        w["q_bits"], wbits, eps, cos.reshape(spec.batch, spec.seq_len_q, 32),
        sin.reshape(spec.batch, spec.seq_len_q, 32), w["k_cache"], w["indices"], w["softmax_scale"],
        w["extra_k_cache"], w["extra_indices"])
    bound, vmax = _flip_bounds(w, wbits, eps, cos, sin)
    print(f"{spec.name}: {np.count_nonzero(bound)} of {bound.size} heads with a query element "
          f"near a bf16 tie, largest bound {bound.max():.2e}", flush=True)
    _check(rec.cpu().numpy(), lse.cpu().numpy().astype(np.float64), rec_ref, lse_ref, out_ref,
           spec.name, bound, vmax)


def test_fused_decode_refuses_64_heads():
    w = make_workload(Spec("fz64", 1, 1, 64, 64, 512), seed=1)
    d = to_dev(w)
    md = mla.get_metadata(1, 1, 64, 64, 0)
    c = torch.ones((1, 1, 32), device="cuda")
    with pytest.raises(mla.MLAError, match="unsupported"):
        mla.sparse_decode_fused(d["q"], torch.ones(512, dtype=torch.bfloat16, device="cuda"), 1e-6, c,
                                c * 0, d["k_cache"], d["indices"], w["softmax_scale"], md)
