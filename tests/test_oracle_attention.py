"""Pins for the oracle's attention, split decode and log-sum-exp merge (CPU only).

Each pin is fixed by the mathematics of softmax attention rather than by the oracle's own code:
closed forms for one and two tokens, identical and duplicated tokens, permutation and -1 padding
invariance, a pure-Python brute force on tiny inputs, a torch float64 softmax on the gathered matrix,
and split-then-merge equal to the unsplit result.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, dequant_fp4_records, dequant_fp8_records, oracle_combine,
                    oracle_decode, oracle_metadata, oracle_split_decode)
from workloads import Spec, encode_fp8_records, make_workload

SCALE = 1.0 / math.sqrt(512)


def _small(seed=0, n_tok=256, h=4, b=2, s=1, topk=40):
    rng = np.random.default_rng(seed)
    cache = encode_fp8_records(rng.standard_normal((n_tok, 512)).astype(np.float32))
    q = torch.randn(b, s, h, 512, generator=torch.Generator().manual_seed(seed)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    idx = np.stack([rng.choice(n_tok, topk, replace=False) for _ in range(b * s)]).reshape(b, s, topk)
    return q, cache, idx.astype(np.int32)


def test_topk_one_returns_the_token():
    q, cache, idx = _small(topk=1)
    out, lse = oracle_decode(q, cache, idx, SCALE)
    qf = bf16_bits_to_f64(q)
    for b in range(2):
        k = dequant_fp8_records(cache[idx[b, 0, 0]][None])[0]
        assert np.array_equal(out[b, 0], np.broadcast_to(k, (4, 512)))
        assert np.allclose(lse[b, 0], SCALE * qf[b, 0] @ k, rtol=0, atol=1e-12)


def test_two_tokens_closed_form():
    q, cache, idx = _small(topk=2)
    out, lse = oracle_decode(q, cache, idx, SCALE)
    qf = bf16_bits_to_f64(q)
    for b in range(2):
        k1, k2 = dequant_fp8_records(cache[idx[b, 0]])
        for h in range(4):
            s1, s2 = SCALE * qf[b, 0, h] @ k1, SCALE * qf[b, 0, h] @ k2
            p1 = 1.0 / (1.0 + math.exp(s2 - s1))                  # sigmoid(s1 - s2)
            big = max(s1, s2)
            assert abs(lse[b, 0, h] - (big + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-12
            assert np.allclose(out[b, 0, h], p1 * k1 + (1 - p1) * k2, rtol=0, atol=1e-12)


def test_identical_tokens_give_log_n_shift():
    q, cache, idx = _small(topk=1)
    n = 7
    rep = np.repeat(idx, n, axis=2)
    out1, lse1 = oracle_decode(q, cache, idx, SCALE)
    outn, lsen = oracle_decode(q, cache, rep, SCALE)
    assert np.allclose(outn, out1, rtol=0, atol=1e-12)
    assert np.allclose(lsen, lse1 + math.log(n), rtol=0, atol=1e-12)


def test_duplicating_every_entry_shifts_lse_by_log2():
    q, cache, idx = _small(topk=33)
    out1, lse1 = oracle_decode(q, cache, idx, SCALE)
    out2, lse2 = oracle_decode(q, cache, np.concatenate([idx, idx[:, :, ::-1]], axis=2), SCALE)
    assert np.allclose(out2, out1, rtol=0, atol=1e-12)
    assert np.allclose(lse2, lse1 + math.log(2.0), rtol=0, atol=1e-12)


def test_permutation_and_padding_invariance():
    q, cache, idx = _small(topk=50, seed=5)
    out, lse = oracle_decode(q, cache, idx, SCALE)
    rng = np.random.default_rng(9)
    perm = idx[:, :, rng.permutation(50)]
    out_p, lse_p = oracle_decode(q, cache, perm, SCALE)
    assert np.allclose(out_p, out, rtol=0, atol=1e-12) and np.allclose(lse_p, lse, atol=1e-12)
    padded = np.full((2, 1, 80), -1, dtype=np.int32)
    for b in range(2):
        pos = np.sort(rng.choice(80, 50, replace=False))
        padded[b, 0, pos] = idx[b, 0]
    padded[0, 0, padded[0, 0] < 0] = -7                            # any negative entry is ignored
    out_q, lse_q = oracle_decode(q, cache, padded, SCALE)
    assert np.allclose(out_q, out, rtol=0, atol=1e-12) and np.allclose(lse_q, lse, atol=1e-12)


def test_empty_row_gives_zero_and_minus_inf():
    q, cache, idx = _small(topk=4)
    idx[1] = -1
    out, lse = oracle_decode(q, cache, idx, SCALE)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))


def test_out_of_pool_index_is_rejected():
    q, cache, idx = _small(topk=4)
    idx[0, 0, 0] = cache.shape[0]
    with pytest.raises(ValueError):
        oracle_decode(q, cache, idx, SCALE)


def test_brute_force_pure_python_tiny():
    q, cache, idx = _small(topk=6, h=2, n_tok=32, seed=11)
    idx[0, 0, 2] = -1
    out, lse = oracle_decode(q, cache, idx, SCALE)
    qf = bf16_bits_to_f64(q)
    for b in range(2):
        toks = [int(t) for t in idx[b, 0] if t >= 0]
        lat = [[float(v) for v in dequant_fp8_records(cache[t][None])[0]] for t in toks]
        for h in range(2):
            qv = [float(v) for v in qf[b, 0, h]]
            sc = [SCALE * sum(a * c for a, c in zip(qv, k)) for k in lat]
            m = max(sc)
            den = sum(math.exp(x - m) for x in sc)
            ref_lse = m + math.log(den)
            ref_out = [sum(math.exp(sc[t] - ref_lse) * lat[t][d] for t in range(len(lat)))
                       for d in range(512)]
            assert abs(lse[b, 0, h] - ref_lse) < 1e-12
            assert max(abs(a - c) for a, c in zip(out[b, 0, h], ref_out)) < 1e-12


def test_torch_float64_softmax_cross_check():
    w = make_workload(Spec("t", 2, 2, 16, 300, 4096, neg="frac5"), seed=21)
    out, lse = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"])
    qf = torch.from_numpy(w["q_bits"].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    for b in range(2):
        for s in range(2):
            sel = w["indices"][b, s]
            sel = sel[sel >= 0]
            lat = torch.from_numpy(dequant_fp8_records(w["k_cache"][sel]))
            sc = w["softmax_scale"] * (qf[b, s] @ lat.T)
            ref_out = torch.softmax(sc, dim=-1) @ lat
            ref_lse = torch.logsumexp(sc, dim=-1)
            assert torch.allclose(torch.from_numpy(out[b, s]), ref_out, rtol=0, atol=1e-12)
            assert torch.allclose(torch.from_numpy(lse[b, s]), ref_lse, rtol=0, atol=1e-12)


def test_extra_cache_is_one_softmax_over_the_union():
    # Records that hold the same latent in both formats: values from the e2m1 set, fp8 scale 1 and
    # fp4 scale 1. Attending over (fp8 A) + (fp4 B) must equal attending over fp8 (A followed by B').
    rng = np.random.default_rng(4)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = rng.choice(mags, size=(40, 512)) * rng.choice([-1.0, 1.0], size=(40, 512))
    c8 = np.zeros((40, 528), dtype=np.uint8)                       # e4m3 data, e8m0 scales 2^0
    c8[:, :512] = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    c8[:, 512:] = 0x7F
    codes = np.searchsorted(mags, np.abs(vals)).astype(np.uint8) | (
        (vals < 0).astype(np.uint8) << 3)                          # e2m1 codes, e4m3 scales 1.0
    c4 = np.zeros((40, 288), dtype=np.uint8)
    c4[:, :256] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    c4[:, 256:] = 0x38
    assert np.array_equal(dequant_fp8_records(c8), dequant_fp4_records(c4))
    q = torch.randn(1, 1, 8, 512, generator=torch.Generator().manual_seed(2)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = np.array([[[3, 7, 11, -1, 20]]], dtype=np.int32)
    bx = np.array([[[5, -1, 30, 31]]], dtype=np.int32)
    out, lse = oracle_decode(q, c8, a, SCALE, extra_k_cache=c4, extra_indices=bx)
    both = np.array([[[3, 7, 11, 20, 5, 30, 31]]], dtype=np.int32)
    out_ref, lse_ref = oracle_decode(q, c8, both, SCALE)
    assert np.allclose(out, out_ref, rtol=0, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)


@pytest.mark.parametrize("parts,min_tiles,extra", [(7, 1, 0), (5, 2, 0), (16, 1, 70), (5, 3, 130)])
def test_split_then_merge_equals_unsplit(parts, min_tiles, extra):
    spec = Spec("s", 3, 2, 8, 200, 2048, extra_topk=extra, extra_tokens_per_seq=1024 if extra else 0,
                neg="tail10")
    w = make_workload(spec, seed=parts * 10 + min_tiles)
    sched, split_ptr, _ = oracle_metadata(3, 2, 200, extra, parts, min_tiles)
    po, pl = oracle_split_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"], sched,
                                 split_ptr, w["extra_k_cache"], w["extra_indices"])
    out_c, lse_c = oracle_combine(po, pl, split_ptr)
    out, lse = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"],
                             w["extra_k_cache"], w["extra_indices"])
    assert np.allclose(out_c.reshape(out.shape), out, rtol=0, atol=1e-12)
    assert np.allclose(lse_c.reshape(lse.shape), lse, rtol=0, atol=1e-12)
    assert np.diff(split_ptr).max() > 1                            # some row really split


def test_combine_closed_form_and_empty_splits():
    o = np.zeros((4, 1, 512))
    o[0, 0, :] = 1.0
    o[1, 0, :] = 3.0
    o[2, 0, :] = 5.0
    lse = np.array([[math.log(1.0)], [math.log(3.0)], [-np.inf], [-np.inf]])
    split_ptr = np.array([0, 3, 4])                                # row0: 3 splits, row1: 1 (empty)
    out, l = oracle_combine(o, lse, split_ptr)
    # weights 1 : 3 : 0 -> out = (1*1 + 3*3) / 4 = 2.5, lse = log 4
    assert np.allclose(out[0, 0], 2.5, atol=1e-15) and abs(l[0, 0] - math.log(4.0)) < 1e-15
    assert np.all(out[1] == 0) and np.isneginf(l[1, 0])
