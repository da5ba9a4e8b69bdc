"""The build-time MFMA wait-state check (sparse_mla_decode_get_amd/asm_check.py) on small
hand-written gfx950 assembly snippets: each rule must fire on a violating snippet and stay quiet on
the corrected one."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", "sparse_mla_decode_get_amd"))
import asm_check  # noqa: E402

MFMA = "v_mfma_f32_32x32x16_bf16"


def _kernel(body):
    return "_Zk:\n" + "\n".join("\t" + l for l in body) + "\n\ts_endpgm\n"


def _problems(body):
    text = _kernel(body)
    assert asm_check.kernels(text, "_Zk") == ["_Zk"]
    return asm_check.check(text, "_Zk")


def test_valu_write_then_mfma_read_needs_two_wait_states():
    bad = ["v_mov_b32_e32 v4, 0", f"{MFMA} v[32:47], v[4:7], v[8:11], 0"]
    good = ["v_mov_b32_e32 v4, 0", "s_nop 1", f"{MFMA} v[32:47], v[4:7], v[8:11], 0"]
    assert any("VALU write" in p for p in _problems(bad))
    assert _problems(good) == []


def test_mfma_result_read_by_valu_needs_twelve_wait_states():
    bad = [f"{MFMA} v[0:15], v[16:19], v[20:23], 0", "s_nop 9", "v_add_f32_e32 v30, v0, v1"]
    good = [f"{MFMA} v[0:15], v[16:19], v[20:23], 0", "s_nop 11", "v_add_f32_e32 v30, v0, v1"]
    assert any("MFMA result used" in p for p in _problems(bad))
    assert _problems(good) == []


def test_chained_accumulator_is_forwarded():
    body = [f"{MFMA} v[0:15], v[16:19], v[20:23], 0", f"{MFMA} v[0:15], v[24:27], v[28:31], v[0:15]"]
    assert _problems(body) == []


def test_result_overlapping_an_a_or_b_operand_is_rejected():
    assert any("overlaps" in p for p in _problems([f"{MFMA} v[0:15], v[16:19], v[0:3], 0"]))
    assert any("overlaps" in p for p in _problems([f"{MFMA} v[0:15], v[12:15], v[20:23], 0"]))
    assert _problems([f"{MFMA} v[0:15], v[16:19], v[20:23], 0"]) == []


def test_m0_outside_inline_asm_is_reported():
    text = ("_Zk:\n\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v[0:1], off\n\t;;#ASMEND\n"
            "\ts_mov_b32 m0, -1\n\tds_write_b32 v0, v1\n\ts_endpgm\n")
    probs = asm_check.m0_outside_inline_asm(text, "_Zk")
    assert len(probs) == 1 and "s_mov_b32 m0, -1" in probs[0]
    assert asm_check.m0_outside_inline_asm(text.replace("\ts_mov_b32 m0, -1\n", ""), "_Zk") == []
