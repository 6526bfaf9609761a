"""The build's MFMA result-hazard gate: it must flag an early read or write
of an MFMA's destination registers, and pass code that waits long enough or
chains accumulations on the same registers."""
import os

import pytest

from mla_paged_kv_05_amd import build

HDR = "0000000000001000 <k>:\n"


def _lines(*insts):
    return HDR + "".join(f"\t{s}   // 000000001000: 00000000\n" for s in insts)


MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"


def test_read_right_after_mfma_is_flagged():
    h = build.mfma_hazards(_lines(MFMA, "v_accvgpr_read_b32 v20, a3"))
    assert len(h) == 1 and "v_accvgpr_read_b32" in h[0]


def test_write_of_accumulator_is_flagged():
    h = build.mfma_hazards(_lines(MFMA, "s_nop 7", "v_accvgpr_write_b32 a15, v2"))
    assert len(h) == 1


def test_enough_nops_pass():
    assert build.mfma_hazards(_lines(MFMA, "s_nop 7", "s_nop 7", "s_nop 1",
                                     "v_accvgpr_read_b32 v20, a3")) == []


def test_counted_instructions_are_wait_states():
    filler = [f"v_add_u32 v{30 + i}, v1, v2" for i in range(build.MFMA_RESULT_WAIT)]
    assert build.mfma_hazards(_lines(MFMA, *filler, "v_accvgpr_read_b32 v20, a3")) == []
    assert len(build.mfma_hazards(_lines(MFMA, *filler[:-1], "v_accvgpr_read_b32 v20, a3"))) == 1


def test_chained_accumulation_is_exempt():
    assert build.mfma_hazards(_lines(MFMA, MFMA)) == []


def test_other_accumulator_overlap_is_flagged():
    h = build.mfma_hazards(_lines(MFMA, "v_mfma_f32_32x32x16_bf16 a[16:31], v[4:7], v[8:11], a[8:23]"))
    assert len(h) == 1


def test_unrelated_registers_pass():
    assert build.mfma_hazards(_lines(MFMA, "v_accvgpr_read_b32 v20, a16", "v_mov_b32 v0, v1")) == []


def test_branch_ends_tracking():
    assert build.mfma_hazards(_lines(MFMA, "s_cbranch_scc1 65", "v_accvgpr_read_b32 v20, a3")) == []


def test_vgpr_accumulator_ranges():
    m = "v_mfma_f32_32x32x16_f16 v[0:15], v[114:117], v[18:21], 0"
    assert len(build.mfma_hazards(_lines(m, "v_exp_f32 v3, v5"))) == 1
    assert build.mfma_hazards(_lines(m, "v_exp_f32 v16, v17")) == []


def test_built_library_has_no_hazards():
    obj = os.path.join(build.ROOT, "_build", "mla_kernels.hip.o")
    if not os.path.exists(obj):
        pytest.skip("library not built in this tree")
    assert build.check_hazards(obj) == []
