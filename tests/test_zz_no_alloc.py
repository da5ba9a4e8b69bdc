"""The allocation-free decode entry point (mla_sparse_decode_noalloc), called through the C ABI.

It runs the same kernels as mla_sparse_decode with its split partials in the library's fixed device
array instead of a caller workspace. Two calls in a row, the second on a smaller input (the array
keeps the first call's contents), each compared with mla_sparse_decode on the same inputs (identical
bits: same kernels, same schedule) and with the oracle at the usual tolerances; and the refusal of a
schedule whose partials would not fit.
"""
import ctypes

import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import oracle_decode
from workloads import Spec, make_workload
from tests.gpu_helpers import check_rows, to_dev

pytestmark = pytest.mark.gpu

NOALLOC_BYTES = 72 << 20
SCRATCH_LIMIT = -6


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(lib, d, w, md, out, lse):
    b, s, h, _ = d["q"].shape
    xc, xi = d.get("extra_k_cache"), d.get("extra_indices")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.mla_sparse_decode_noalloc(
        _p(d["q"]), _p(d["k_cache"]), d["k_cache"].numel() // 528, _p(d["indices"]),
        d["indices"].shape[2], _p(xc), 0 if xc is None else xc.numel() // 288, _p(xi),
        0 if xi is None else xi.shape[2], b, s, h, ctypes.c_float(w["softmax_scale"]),
        _p(md.sched), _p(md.split_ptr), md.num_parts, _p(out), _p(lse), stream)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(order):
    lib = mla.load_library()
    cases = [
        # 128-head kernel, fp32 partials; rows split over 37 parts
        (Spec("na_large", 4, 2, 128, 1500, 8192, values="spread", neg="tail10"), 37),
        # 64-head kernel with the fp4 extra cache, bf16 partials; smaller
        (Spec("na_small", 2, 1, 64, 300, 2048, extra_topk=70, extra_tokens_per_seq=1024,
              neg="frac5"), 7),
    ]
    for k, (spec, parts) in enumerate(cases):
        w = make_workload(spec, seed=71 + k)
        d = to_dev(w)
        extra = spec.extra_topk
        md = mla.get_metadata(spec.batch, spec.seq_len_q, spec.h_q, spec.topk, extra, num_parts=parts)
        assert md.workspace is not None                       # rows really are split
        assert md.workspace.numel() <= NOALLOC_BYTES
        ref_o, ref_l = mla.sparse_decode(d["q"], d["k_cache"], d["indices"], w["softmax_scale"], md,
                                         d.get("extra_k_cache"), d.get("extra_indices"))
        out = torch.full_like(ref_o, 7.0)
        lse = torch.full_like(ref_l, 7.0)
        rc = _noalloc(lib, d, w, md, out, lse)
        assert rc == 0, mla.error_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"{spec.name}: output differs from mla_sparse_decode"
        assert torch.equal(lse, ref_l), f"{spec.name}: lse differs from mla_sparse_decode"
        o_ref, l_ref = oracle_decode(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"],
                                     w["extra_k_cache"], w["extra_indices"])
        check_rows(out, lse, o_ref, l_ref, spec.name)


def test_noalloc_refuses_a_schedule_beyond_the_fixed_array():
    """Partials of 8 rows x 128 heads over 4096 parts need about 1 GiB: refused with
    MLA_ERR_SCRATCH_LIMIT before any device work (dummy, never dereferenced addresses)."""
    lib = mla.load_library()
    batch, seq, h_q, topk, parts = 8, 1, 128, 131072, 4096
    assert mla.workspace_bytes(batch, seq, h_q, topk, 0, parts) > NOALLOC_BYTES
    a = 1 << 20
    q, kc, idx, sched, sp, out, lse = (a * i for i in range(1, 8))
    rc = lib.mla_sparse_decode_noalloc(q, kc, 1 << 20, idx, topk, None, 0, None, 0, batch, seq, h_q,
                                       ctypes.c_float(0.04), sched, sp, parts, out, lse, None)
    assert rc == SCRATCH_LIMIT
    assert "MLA_NOALLOC_SCRATCH_BYTES" in mla.error_string(rc)
