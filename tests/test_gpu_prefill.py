"""GPU parity of sparse prefill (mla_sparse_prefill): many query rows of one sequence, each with its
own selection over the quantized cache, no metadata and no split. Compared with the oracle on every
row, and with the decode path on the same rows (identical bits: one row per part runs the same
per-row kernel work)."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import oracle_decode, oracle_decode_rows
from workloads import Spec, make_workload
from tests.gpu_helpers import check_rows, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    Spec("pf_h128", 1, 300, 128, 512, 8192, values="spread", neg="tail10"),
    Spec("pf_h64", 1, 257, 64, 700, 8192, neg="frac5"),
    Spec("pf_h16_mixed", 1, 100, 16, 256, 4096, extra_topk=96, extra_tokens_per_seq=2048,
         neg="frac5"),
    Spec("pf_h128_mixed", 1, 64, 128, 130, 2048, extra_topk=70, extra_tokens_per_seq=1024),
    Spec("pf_h200", 1, 40, 200, 100, 2048),
    Spec("pf_few_rows", 1, 3, 128, 64, 512),
    Spec("pf_empty_rows", 1, 50, 64, 80, 1024, neg="all"),
]


def _prefill(w):
    d = to_dev(w)
    s = w["spec"].seq_len_q
    q = d["q"].reshape(s, w["spec"].h_q, 512)
    xi = d.get("extra_indices")
    out, lse = mla.sparse_prefill(q, d["k_cache"], d["indices"].reshape(s, -1), w["softmax_scale"],
                                  d.get("extra_k_cache"), None if xi is None else xi.reshape(s, -1))
    torch.cuda.synchronize()
    return out, lse, d


@pytest.mark.parametrize("spec", CASES, ids=[c.name for c in CASES])
def test_prefill_matches_oracle_and_decode(spec):
    w = make_workload(spec, seed=91)
    out, lse, d = _prefill(w)
    ref_out, ref_lse = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"],
                                     w["extra_k_cache"], w["extra_indices"])
    check_rows(out, lse, ref_out, ref_lse, spec.name)
    # the decode path with one whole row per part runs the same per-row work
    md = mla.get_metadata(1, spec.seq_len_q, spec.h_q, spec.topk, spec.extra_topk,
                          num_parts=spec.seq_len_q)
    o2, l2 = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md,
                               d.get("extra_k_cache"), d.get("extra_indices"))
    torch.cuda.synchronize()
    assert torch.equal(out, o2.reshape(out.shape)) and torch.equal(lse, l2.reshape(lse.shape))


def test_prefill_large_every_row():
    """4096 query rows of 128 heads over a 65536-token cache, 2048 selected per row (the last 0-10%
    ignored), spread values: 16 rows per part; every row against the oracle."""
    spec = Spec("pf_large", 1, 4096, 128, 2048, 65536, values="spread", neg="tail10")
    w = make_workload(spec, seed=93)
    out, lse, _ = _prefill(w)
    o = out.reshape(4096, 128, 512)
    l = lse.reshape(4096, 128)
    for r0 in range(0, 4096, 256):
        rows = list(range(r0, r0 + 256))
        ro, rl = oracle_decode_rows(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"], rows)
        check_rows(o[rows], l[rows], ro, rl, f"pf_large rows {r0}..")


def test_prefill_accepts_one_kv_head_axis():
    spec = Spec("pf_axis", 1, 20, 64, 100, 1024)
    w = make_workload(spec, seed=95)
    d = to_dev(w)
    q = d["q"].reshape(20, 64, 512)
    o1, l1 = mla.sparse_prefill(q, d["k_cache"], d["indices"].reshape(20, 1, 100), w["softmax_scale"])
    o2, l2 = mla.sparse_prefill(q, d["k_cache"], d["indices"].reshape(20, 100), w["softmax_scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
