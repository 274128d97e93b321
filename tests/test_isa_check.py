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


# the read's wait is on one path only: the branch skips it
BRANCH_SKIPS_WAIT = """
kern:
;;#ASMSTART
	ds_read_b128 v[4:7], v1 offset:0
;;#ASMEND
	s_cbranch_scc1 .LBB0_2
;;#ASMSTART
	s_waitcnt lgkmcnt(0)
;;#ASMEND
.LBB0_2:
	v_mov_b32_e32 v5, 0
	s_endpgm
"""
# the wait is on both paths
WAIT_ON_BOTH = BRANCH_SKIPS_WAIT.replace(""".LBB0_2:
	v_mov_b32_e32 v5, 0""", """	s_branch .LBB0_3
.LBB0_2:
	s_waitcnt lgkmcnt(0)
.LBB0_3:
	v_mov_b32_e32 v5, 0""")
# the use comes later in the text than the read, but control flow reaches it only
# through a block (laid out after it) that waits
LAYOUT = """
kern:
;;#ASMSTART
	ds_read_b128 v[4:7], v1 offset:0
;;#ASMEND
	s_branch .LBB0_2
.LBB0_1:
	v_mov_b32_e32 v6, 0
	s_endpgm
.LBB0_2:
;;#ASMSTART
	s_waitcnt lgkmcnt(0)
;;#ASMEND
	s_branch .LBB0_1
"""


def test_control_flow():
    assert check_isa.check_text(BRANCH_SKIPS_WAIT)
    assert check_isa.check_text(WAIT_ON_BOTH) == []
    assert check_isa.check_text(LAYOUT) == []


def test_register_ranges():
    assert check_isa.regs_of("v[4:7], v1, s3") == {1, 4, 5, 6, 7}


def test_kernel_sources_have_no_hazards():
    assert check_isa.check_sources() == []
