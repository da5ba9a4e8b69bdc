"""Pins of the fused-decode oracle's steps (oracle/fused.py): the RMSNorm against torch's
rms_norm, the rotation against complex multiplication, the bfloat16 rounding against torch's cast,
and the composition against the plain decode when the norm and rotation are identities."""
import math

import numpy as np
import torch

from oracle import encode_fp8_records, oracle_decode
from oracle.fused import oracle_fused_decode, rms_norm, rope, round_bf16


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3, 5, 512)) * np.exp2(rng.uniform(-3, 3, (3, 5, 1)))
    w = 1 + 0.1 * rng.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(q), (512,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(rms_norm(q, w, 1e-6), ref.numpy(), rtol=1e-13, atol=0)
    # closed form: a constant row c becomes c / sqrt(c^2 + eps) * w
    c = np.full(512, 3.0)
    assert np.allclose(rms_norm(c, w, 0.5), 3.0 / math.sqrt(9.5) * w, rtol=1e-15)


def test_rope_is_complex_rotation_of_the_last_64_dims():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 512))
    ang = rng.uniform(-10, 10, (4, 32))
    y = rope(x, np.cos(ang), np.sin(ang))
    z = (x[:, 448::2] + 1j * x[:, 449::2]) * np.exp(1j * ang)
    assert np.array_equal(y[:, :448], x[:, :448])
    assert np.allclose(y[:, 448::2], z.real, atol=1e-13) and np.allclose(y[:, 449::2], z.imag, atol=1e-13)
    back = rope(y, np.cos(ang), np.sin(ang), conjugate=True)
    assert np.allclose(back, x, atol=1e-13)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_round_bf16_matches_torch_and_ties_go_to_even():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(100000) * np.exp2(rng.uniform(-100, 100, 100000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x32.astype(np.float64)), ref)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133 * 2.5])
    assert np.array_equal(round_bf16(ties), [1.0, 1 + 2 ** -6, -1.0, 2 ** -132])   # subnormal tie -> even


def test_fused_reduces_to_the_plain_decode_with_identity_norm_and_rotation():
    from workloads import Spec, make_workload
    w = make_workload(Spec("fz", 2, 1, 8, 100, 1024, neg="frac5"), seed=3)
    one = np.full(512, 0x3F80, dtype=np.uint16)                  # bf16 1.0
    cos = np.ones((2, 1, 32), np.float32)
    sin = np.zeros((2, 1, 32), np.float32)
    rec, lse, out_r = oracle_fused_decode(w["q_bits"], one, 0.0, cos, sin, w["k_cache"],
                                          w["indices"], w["softmax_scale"])
    from oracle import bf16_bits_to_f64
    q = bf16_bits_to_f64(w["q_bits"])
    qn = round_bf16(q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True)))
    o, l = oracle_decode(qn, w["k_cache"], w["indices"], w["softmax_scale"])
    assert np.array_equal(lse, l) and np.array_equal(out_r, o)
    assert np.array_equal(rec, encode_fp8_records(o.reshape(-1, 512)).reshape(rec.shape))
