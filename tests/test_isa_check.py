"""The build-time check for inline-asm LDS reads (exact_io_aware_49_amd/check_isa.py)."""

import pytest

from exact_io_aware_49_amd import check_isa

GOOD = """
kern:
;;#ASMSTART
	ds_read_b128 v[4:7], v1 offset:0
;;#ASMEND
	v_add_u32_e32 v9, v2, v3
;;#ASMSTART
	s_waitcnt lgkmcnt(0)
;;#ASMEND
	v_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], v[8:11], v[16:31]
"""

BAD_COPY = GOOD.replace("	v_add_u32_e32 v9, v2, v3", "	v_mov_b64_e32 v[12:13], v[4:5]")
BAD_OVERWRITE = GOOD.replace("	v_add_u32_e32 v9, v2, v3", "	v_mov_b32_e32 v6, 0")
PARTIAL_WAIT = GOOD.replace("	v_add_u32_e32 v9, v2, v3", "	s_waitcnt lgkmcnt(1)\n	v_mov_b32_e32 v12, v5")


def test_clean_sequence_passes():
    assert check_isa.check_text(GOOD) == []


@pytest.mark.parametrize("text", [BAD_COPY, BAD_OVERWRITE, PARTIAL_WAIT])
def test_premature_use_is_flagged(text):
    assert check_isa.check_text(text)


def test_register_ranges():
    assert check_isa.regs_of("v[4:7], v1, s3") == {1, 4, 5, 6, 7}


def test_kernel_sources_have_no_hazards():
    assert check_isa.check_sources() == []
