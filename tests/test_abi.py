"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and its
host-side logic (part count, workspace size, argument errors) agrees with the oracle's partition."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_mla_decode_get_amd as mla
from oracle import oracle_metadata, part_count, tiles_per_row

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.library_path()):
        pytest.skip("libmla.so not built")
    return mla.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 8
    raw = ctypes.CDLL(mla.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(mla.error_string(code), str) and mla.error_string(code)


@pytest.mark.parametrize("batch,seq,topk,extra,parts,min_tiles",
                         [(1, 1, 128, 0, 256, 1), (128, 2, 2048, 0, 256, 1), (32, 1, 2048, 0, 512, 1),
                          (64, 1, 2048, 512, 512, 4), (8, 1, 131072, 0, 256, 1), (3, 2, 150, 70, 7, 2),
                          (2, 1, 0, 0, 4, 1)])
def test_part_count_and_workspace_match_oracle(lib, batch, seq, topk, extra, parts, min_tiles):
    p = mla.metadata_parts(batch, seq, 64, topk, extra, parts, min_tiles)
    assert p == part_count(batch * seq, tiles_per_row(topk, extra), parts, min_tiles)
    _, split_ptr, p_oracle = oracle_metadata(batch, seq, topk, extra, parts, min_tiles) \
        if batch * seq * tiles_per_row(topk, extra) <= 4096 else (None, None, p)
    ws = mla.workspace_bytes(batch, seq, 64, topk, extra, p)
    if split_ptr is not None:
        split = bool(np.any(np.diff(split_ptr) > 1))
        assert (ws > 0) == split
        if split:
            slots = batch * seq + p - 1
            assert ws >= slots * 64 * 512 * 2 + slots * 64 * 4      # bf16 partials, fp32 lse


def test_headline_schedule_needs_no_workspace(lib):
    p = mla.metadata_parts(128, 2, 128, 2048, 0, 256, 1)
    assert p == 256 and mla.workspace_bytes(128, 2, 128, 2048, 0, p) == 0


def test_argument_errors_before_any_device_work(lib):
    L = lib
    null = None
    # decode with null pointers -> invalid argument (checked on the host, nothing enqueued)
    rc = L.mla_sparse_decode(null, null, 0, null, 16, null, 0, null, 0, 1, 1, 16, 0.1, null, null, 1,
                             null, 0, null, null, null)
    assert rc == -1
    rc = L.mla_sparse_decode(null, null, 0, null, -1, null, 0, null, 0, 1, 1, 16, 0.1, null, null, 1,
                             null, 0, null, null, null)
    assert rc == -1
    assert L.mla_combine(null, null, null, 4, 16, null, null, null) == -1
    assert L.mla_dequant_records(null, 100, null, 4, null, null) == -2
    assert L.mla_validate_indices(null, 4, 10, null, null) == -1
    out = ctypes.c_int(0)
    assert L.mla_metadata_parts(1, 1, 16, 128, 0, 4, 0, ctypes.byref(out)) == -1   # min_tiles 0
    assert L.mla_metadata_parts(-1, 1, 16, 128, 0, 4, 1, ctypes.byref(out)) == -1
    assert L.mla_get_metadata(1, 1, 16, 128, 0, 4, 1, null, 4, null, ctypes.byref(out), null) == -1
    # zero rows is a no-op
    assert L.mla_sparse_decode(null, null, 0, null, 16, null, 0, null, 0, 0, 1, 16, 0.1, null, null,
                               1, null, 0, null, null, null) == 0


def test_resource_report_parser():
    from sparse_mla_decode_get_amd.build import _parse_resources
    text = ("x.hip:1:1: remark: Function Name: kern [-Rpass]\n"
            "x.hip:1:1: remark:     VGPRs: 12 [-Rpass]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass]\n"
            "x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass]\n")
    r = _parse_resources(text)
    assert r == {"kern": {"VGPRs": 12, "ScratchSize [bytes/lane]": 0, "VGPRs Spill": 3}}


@pytest.mark.parametrize("batch,seq,h_q,topk,extra,min_tiles,expected", [
    (32, 1, 64, 2048, 0, 1, 256),        # 1024 units: at least 4 per part caps the 512 default
    (64, 1, 64, 2048, 512, 1, 256),      # 2560 units: the default (one part per CU) stands
    (128, 2, 128, 2048, 0, 1, 256),      # headline: one part per CU and row
    (1, 1, 16, 128, 0, 1, 1),            # 2 units: a single part
    (32, 1, 64, 2048, 0, 8, 128),        # a larger caller minimum is kept
])
def test_automatic_part_count_keeps_four_units_per_part(lib, batch, seq, h_q, topk, extra,
                                                       min_tiles, expected):
    # num_parts = 0 selects the device default (256 CUs on MI355X, also the fallback without a
    # device): one part per CU divided by the head groups, with at least max(min_tiles_per_part, 4)
    # units per part
    p = mla.metadata_parts(batch, seq, h_q, topk, extra, 0, min_tiles)
    groups = -(-h_q // (128 if h_q > 64 else 64))
    assert p == part_count(batch * seq, tiles_per_row(topk, extra), 256 // groups, max(min_tiles, 4))
    assert p == expected


def test_host_checks_reject_bad_workspace_scale_and_alignment(lib):
    """These checks run on the host before anything is enqueued, so dummy (never dereferenced)
    device addresses suffice: a split schedule without enough workspace, a non-finite softmax
    scale and a misaligned q are refused with their documented codes."""
    L = lib
    batch, seq, h_q, topk, parts = 2, 1, 64, 256, 5          # 8 units over 5 parts: rows split
    p = mla.metadata_parts(batch, seq, h_q, topk, 0, parts, 1)
    need = mla.workspace_bytes(batch, seq, h_q, topk, 0, p)
    assert need > 0
    a = 1 << 20                                              # dummy 256-byte aligned addresses
    q, kc, idx, sched, sp, out, lse, ws = (a * i for i in range(1, 9))
    tokens = 4096

    def decode(scale=0.04, qp=q, ws_ptr=ws, ws_bytes=need):
        return L.mla_sparse_decode(qp, kc, tokens, idx, topk, None, 0, None, 0, batch, seq, h_q, scale,
                                   sched, sp, p, ws_ptr, ws_bytes, out, lse, None)

    assert decode(ws_ptr=None) == -3                         # MLA_ERR_WORKSPACE: none given
    assert decode(ws_bytes=need - 1) == -3                   # too small
    assert decode(ws_ptr=ws + 16) == -3                      # not 256-byte aligned
    assert decode(scale=float("inf")) == -1                  # MLA_ERR_INVALID_ARG
    assert decode(scale=float("nan")) == -1
    assert decode(scale=0.0) == -1                           # the scale must be positive
    assert decode(scale=-0.0) == -1
    assert decode(scale=-0.04) == -1
    assert decode(scale=-float("inf")) == -1
    assert decode(qp=q + 2) == -1                            # q not 16-byte aligned


def test_shapes_whose_partition_could_overflow_are_refused(lib):
    """rows * units_per_row is bounded (2^40) so that the partition's products p * U stay inside
    int64 for every allowed part count; larger shapes are refused before any device work."""
    out = ctypes.c_int(0)
    # 2^24 rows x 2^22 units per row = 2^46 units
    assert lib.mla_metadata_parts(1 << 24, 1, 16, 1 << 28, 0, 4, 1, ctypes.byref(out)) == -2
    assert mla.workspace_bytes(1 << 24, 1, 16, 1 << 28, 0, 4) == 0
    # just inside the bound: 2^24 rows x 2^16 units
    assert lib.mla_metadata_parts(1 << 24, 1, 16, 1 << 22, 0, 4, 1, ctypes.byref(out)) == 0
    assert out.value == 4


def test_check_indices_argument_errors(lib):
    assert lib.mla_check_indices(None, 4, 10, None, None) == -1
    assert lib.mla_check_indices(None, -1, 10, 1 << 20, None) == -1


def test_prefill_argument_errors(lib):
    null = None
    # null q / cache / indices -> invalid argument; zero rows -> no-op; bad scale -> invalid
    assert lib.mla_sparse_prefill(null, 4, 64, null, 0, null, 16, null, 0, null, 0, 0.04, null, null,
                                  null) == -1
    assert lib.mla_sparse_prefill(null, 0, 64, null, 0, null, 16, null, 0, null, 0, 0.04, null, null,
                                  null) == 0
    a = 1 << 20
    assert lib.mla_sparse_prefill(a, 4, 64, 2 * a, 100, 3 * a, 16, null, 0, null, 0, -1.0, 4 * a,
                                  5 * a, null) == -1
    assert lib.mla_sparse_prefill(a + 2, 4, 64, 2 * a, 100, 3 * a, 16, null, 0, null, 0, 0.04,
                                  4 * a, 5 * a, null) == -1
