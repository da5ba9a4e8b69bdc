"""GPU parity of the cache writer (mla_quantize_records) with the oracle's encoder: bit-exact records
on random values over a wide range, on blocks built to hit every rounding tie, on saturating fp4
blocks, on zeros, negative zeros and bf16 subnormals; scatter into a pool by slot, with skipped
slots; and a decode over records the writer produced."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_get_amd as mla
from oracle import E2M1, E4M3, encode_fp4_records, encode_fp8_records, oracle_decode
from tests.gpu_helpers import check_rows

pytestmark = pytest.mark.gpu


def _bf16_tensor(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _values(t):
    return t.to(torch.float64).numpy()


def _write(xb, rec_bytes):
    got = mla.quantize_records(xb.cuda(), rec_bytes)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _random_rows(n, seed, lo=-30, hi=30):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)) * np.exp2(rng.uniform(lo, hi, (n, 32, 1))).repeat(16, 2).reshape(n, 512)
    return _bf16_tensor(x)


@pytest.mark.parametrize("rec_bytes", [528, 288])
def test_random_values_bit_exact(rec_bytes):
    xb = _random_rows(2048, 1 + rec_bytes, -40, 40) if rec_bytes == 528 else _random_rows(2048, 2, -12, 9)
    enc = encode_fp8_records if rec_bytes == 528 else encode_fp4_records
    assert np.array_equal(_write(xb, rec_bytes), enc(_values(xb)))


def test_fp8_every_tie_and_the_block_limits():
    pos = E4M3[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                     # 126 exact e4m3 ties
    rows = []
    for k in (-20, 0, 7, 60):
        for sign in (1.0, -1.0):
            for start in range(0, len(mids), 31):
                r = np.zeros(512)
                for b in range(16):                     # every block: amax 448 * 2^k, then ties
                    blk = np.zeros(32)
                    blk[0] = 448.0
                    m = mids[(start + np.arange(31) + b) % len(mids)]
                    blk[1:] = sign * m
                    r[32 * b:32 * b + 32] = blk * 2.0 ** k
                rows.append(r)
    # the limits: a block at exactly 448 * 2^k, one just above (scale 2^(k+1)), an all-zero block,
    # negative zeros, bf16 subnormals (k clipped to -127), the largest bf16 values
    r = np.zeros(512)
    r[0:32] = 448.0
    r[32:64] = np.linspace(-449.0, 449.0, 32)
    r[96:128] = -0.0
    r[128:160] = 2.0 ** -133 * np.arange(32)
    r[160:192] = 3.0e38 * np.linspace(-1, 1, 32)
    r[192:224] = 2.0 ** -126 * np.linspace(-1.5, 1.5, 32)
    rows.append(r)
    xb = _bf16_tensor(np.array(rows))
    assert np.array_equal(_values(xb)[:-1], np.array(rows)[:-1])   # the ties are bf16 values
    assert np.array_equal(_write(xb, 528), encode_fp8_records(_values(xb)))


def test_fp4_every_tie_saturation_and_zero_scales():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for s in (1.0, 0.5, 0.375, 2.0 ** -7, 96.0):       # exact e4m3 scales: amax = 6 s
        for sign in (1.0, -1.0):
            r = np.zeros(512)
            for b in range(32):
                blk = np.zeros(16)
                blk[0] = 6.0 * s
                blk[1:8] = sign * mids * s
                blk[8:15] = -sign * mids[::-1] * s
                r[16 * b:16 * b + 16] = blk
            rows.append(r)
    r = np.zeros(512)
    r[0:16] = 6.0 * 1.0625                              # amax / 6 = 1.0625 rounds to 1.0: values saturate
    r[16:32] = np.linspace(-6.375, 6.375, 16)
    r[32:48] = 3000.0 * np.linspace(-1, 1, 16)          # amax / 6 > 448: the scale saturates too
    r[48:64] = 2.0 ** -133 * np.arange(16)              # amax / 6 rounds to 0: scale 1.0
    r[64:80] = -0.0
    rows.append(r)
    xb = _bf16_tensor(np.array(rows))
    assert np.array_equal(_values(xb)[:-1], np.array(rows)[:-1])   # the ties are bf16 values
    got = _write(xb, 288)
    assert np.array_equal(got, encode_fp4_records(_values(xb)))
    assert got[-1, 256] == 0x38 and got[-1, 259] == 0x38 and got[-1, 258] == 0x7E


@pytest.mark.parametrize("rec_bytes", [528, 288])
def test_scatter_by_slot_leaves_other_records_alone(rec_bytes):
    n, pool_tokens = 200, 1000
    xb = _random_rows(n, 5, -8, 8)
    rng = np.random.default_rng(6)
    slots = rng.permutation(pool_tokens)[:n].astype(np.int32)
    slots[[3, 50]] = -1                                  # skipped
    slots[[7]] = pool_tokens + 5                         # past the pool: skipped
    pool = np.full((pool_tokens, rec_bytes), 0xA5, dtype=np.uint8)
    cache = torch.from_numpy(pool.copy()).cuda()
    mla.quantize_records(xb.cuda(), rec_bytes, cache=cache, slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    enc = (encode_fp8_records if rec_bytes == 528 else encode_fp4_records)(_values(xb))
    live = (slots >= 0) & (slots < pool_tokens)
    expect = pool.copy()
    expect[slots[live]] = enc[live]
    assert np.array_equal(got, expect)


def test_decode_over_records_the_writer_produced():
    """Latents written by the GPU writer into a pool, then decoded: the decode matches the oracle
    run on the same bytes, and the bytes are the oracle encoder's."""
    rng = np.random.default_rng(8)
    b, h, topk, pool_tokens = 2, 64, 300, 4096
    lat = _bf16_tensor(rng.standard_normal((b * topk, 512)))
    slots = rng.permutation(pool_tokens)[:b * topk].astype(np.int32)
    cache = torch.zeros((pool_tokens, 528), dtype=torch.uint8, device="cuda")
    mla.quantize_records(lat.cuda(), 528, cache=cache, slots=torch.from_numpy(slots).cuda())
    q = _bf16_tensor(rng.standard_normal((b, 1, h, 512)))
    idx = torch.from_numpy(slots.reshape(b, 1, topk))
    md = mla.get_metadata(b, 1, h, topk, 0)
    out, lse = mla.sparse_decode(q.cuda(), cache, idx.cuda(), 512 ** -0.5, md)
    torch.cuda.synchronize()
    kc = cache.cpu().numpy()
    assert np.array_equal(kc[slots], encode_fp8_records(_values(lat)))
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    ref_out, ref_lse = oracle_decode(q_bits, kc, idx.numpy(), 512 ** -0.5)
    check_rows(out, lse, ref_out, ref_lse, "written cache")
