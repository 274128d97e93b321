"""The build-time checks of the generated assembly around inline asm
(exact_io_aware_49_amd/check_isa.py): LDS reads waited before use, and
matrix-core results not touched by inline asm before they land."""

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
    assert check_isa.anyregs_of("a[0:1], v2, s3") == {("a", 0), ("a", 1), ("v", 2)}


# an inline-asm instruction reads a matrix-core result right after the v_mfma
MFMA_ASM_READ = """
kern:
	v_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], v[8:11], v[16:31]
;;#ASMSTART
	v_max3_f32 v0, v16, v17, v18
;;#ASMEND
	s_endpgm
"""
# enough wait states in between (s_nop N counts N + 1)
MFMA_PADDED = MFMA_ASM_READ.replace(";;#ASMSTART\n\tv_max3", "\ts_nop 15\n\ts_nop 2\n;;#ASMSTART\n\tv_max3")
# one wait state short
MFMA_SHORT = MFMA_ASM_READ.replace(";;#ASMSTART\n\tv_max3", "\ts_nop 15\n\ts_nop 1\n;;#ASMSTART\n\tv_max3")
# a compiler-generated read of the result (padded by the compiler) comes first
MFMA_COMPILER_READ = MFMA_ASM_READ.replace(";;#ASMSTART\n\tv_max3", "\tv_mul_f32_e32 v40, v31, v41\n;;#ASMSTART\n\tv_max3")
# an accumulating v_mfma reading the result is not evidence that it has landed
MFMA_CHAIN = MFMA_ASM_READ.replace(
    ";;#ASMSTART\n\tv_max3", "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[4:7], v[8:11], v[16:31]\n;;#ASMSTART\n\tv_max3")
# the padding sits on one path only: the branch skips it
MFMA_BRANCH = """
kern:
	v_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], v[8:11], v[16:31]
	s_cbranch_scc1 .LBB0_2
	s_nop 15
	s_nop 7
.LBB0_2:
;;#ASMSTART
	v_max3_f32 v0, v16, v17, v18
;;#ASMEND
	s_endpgm
"""
# the destination of an inline-asm LDS read may be a register of the result
MFMA_LDS_DEST = MFMA_ASM_READ.replace("v_max3_f32 v0, v16, v17, v18", "ds_read_b64_tr_b16 v[16:17], v1 offset:0")
# but its address may not
MFMA_LDS_ADDR = MFMA_ASM_READ.replace("v_max3_f32 v0, v16, v17, v18", "ds_read_b64_tr_b16 v[2:3], v16 offset:0")


def test_matrix_core_results_read_by_inline_asm():
    assert check_isa.check_text(MFMA_ASM_READ)
    assert check_isa.check_text(MFMA_PADDED) == []
    assert check_isa.check_text(MFMA_SHORT)
    assert check_isa.check_text(MFMA_COMPILER_READ) == []
    assert check_isa.check_text(MFMA_CHAIN)
    assert check_isa.check_text(MFMA_BRANCH)
    assert check_isa.check_text(MFMA_LDS_DEST) == []
    assert check_isa.check_text(MFMA_LDS_ADDR)


def test_kernel_sources_have_no_hazards():
    assert check_isa.check_sources() == []
