"""The gfx950 assembly of every kernel is free of the MFMA accumulator-input
(SrcC) rewrite hazard described in test_regression_amd/codegen_check.py."""
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
