"""The gfx950 assembly of every kernel is free of the MFMA accumulator-input
(SrcC) rewrite hazard and of the inline-asm wait-state hazards described in
test_regression_amd/codegen_check.py."""
import shutil

import pytest

from test_regression_amd import build, codegen_check


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not __import__("os").path.exists(build.HIPCC),
                    reason="hipcc not available")
def test_no_mfma_srcc_rewrite_hazard():
    res = codegen_check.check_all()
    assert set(res) == {s for s in build.SOURCES if s != "mesa_host.hip"}
    bad = {k: v[:3] for k, v in res.items() if v}
    assert not bad, bad


def test_scanner_flags_the_known_bad_sequence():
    bad = """
    v_mfma_f32_16x16x4_f32 a[20:23], v40, v44, a[16:19]
    s_nop 8
    v_accvgpr_write_b32 a19, 0
    """
    good = """
    v_mfma_f32_16x16x4_f32 a[16:19], v40, v44, a[16:19]
    s_nop 8
    v_accvgpr_write_b32 a19, 0
    """
    assert len(codegen_check.scan_asm(bad)) == 1
    assert codegen_check.scan_asm(good) == []
    # a range write by a load is seen too; a later MFMA's destination is not a hazard
    range_write = bad.replace("v_accvgpr_write_b32 a19, 0", "ds_read_b128 a[16:19], v2")
    later_mfma = bad.replace("v_accvgpr_write_b32 a19, 0", "v_mfma_f32_16x16x4_f32 a[16:19], v41, v45, 0")
    assert len(codegen_check.scan_asm(range_write)) == 1
    assert codegen_check.scan_asm(later_mfma) == []


def test_scanner_flags_inline_asm_hazards():
    mfma_reads_too_soon = """
    ;;#ASMSTART
    v_fma_mixlo_f16 v10, v3, v4, 0
    v_fma_mixhi_f16 v10, v3, v5, 0
    ;;#ASMEND
    s_nop 0
    v_mfma_f32_16x16x32_f16 a[0:3], v[20:23], v[8:11], a[0:3]
    """
    waited = mfma_reads_too_soon.replace("s_nop 0", "s_nop 1")
    reads_mfma_result = """
    v_mfma_f32_16x16x32_f16 v[4:7], v[20:23], v[24:27], 0
    v_add_f32_e32 v30, v31, v32
    ;;#ASMSTART
    v_fma_mixlo_f16 v10, v3, v5, 0
    ;;#ASMEND
    """
    rewritten_first = reads_mfma_result.replace("v_add_f32_e32 v30, v31, v32", "v_mov_b32_e32 v5, 0")
    assert len(codegen_check.scan_inline_asm(mfma_reads_too_soon)) == 1
    assert codegen_check.scan_inline_asm(waited) == []
    assert len(codegen_check.scan_inline_asm(reads_mfma_result)) == 1
    assert codegen_check.scan_inline_asm(rewritten_first) == []


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not __import__("os").path.exists(build.HIPCC),
                    reason="hipcc not available")
def test_headline_cg_loops_keep_lds_reads_in_flight():
    # each wave's CG iteration in the d = 128, 64-token, bf16-key kernel waits
    # for all its LDS reads at most a dozen times (6-7 with reads kept in
    # flight; 27-29 when the compiler waits on each read as it is issued,
    # about 11% slower for that wave)
    text = codegen_check.compile_asm("cg_output_bf16.hip")
    loops = codegen_check.loop_lds_waits(text, "_ZN4mesa12cg_h2_kernelILi128ELi64ENS_6bf16_tEEEv")
    assert sorted(m for m, _ in loops) == [120, 120, 128, 128], loops
    assert all(w <= 12 for _, w in loops), loops


def test_loop_wait_counter():
    text = """_ZN4mesa3fooEv:
    s_mov_b32 s0, 0
.LBB0_1:
    ds_read_b128 v[0:3], v4
    s_waitcnt lgkmcnt(0)
    v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[0:3], a[0:3]
    v_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[0:3], a[4:7]
    s_waitcnt lgkmcnt(1)
    s_cbranch_scc1 .LBB0_1
    s_endpgm
_ZN4mesa3barEv:
.LBB1_1:
    v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[0:3], a[0:3]
    s_cbranch_scc1 .LBB1_1
"""
    assert codegen_check.loop_lds_waits(text, "_ZN4mesa3fooEv", min_mfma=1) == [(2, 1)]
    assert codegen_check.loop_lds_waits(text, "_ZN4mesa3barEv", min_mfma=1) == [(1, 0)]
    assert codegen_check.loop_lds_waits(text, "_ZN4mesa3fooEv", min_mfma=3) == []
