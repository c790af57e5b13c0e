"""The build-time check for wait states before inline-asm direct-to-LDS loads.

The fixtures restate, in miniature, the instruction order the compiler produced
for an SGPR-addressed load: a v_readfirstlane forming the SGPR base directly
before the load (which read a stale base and faulted), and the same sequence
with the wait states the asm now carries.
"""

from fp8_kv_paged_attn_amd import asm_hazards

STALE_BASE = """
	v_lshl_add_u64 v[2:3], s[22:23], 0, v[2:3]
	s_mov_b32 m0, s10
	v_readfirstlane_b32 s9, v3
	v_readfirstlane_b32 s8, v2
	;;#ASMSTART
	global_load_lds_dwordx4 v104, s[8:9]
	;;#ASMEND
	s_add_i32 m0, s10, 0x400
	;;#ASMSTART
	global_load_lds_dwordx4 v102, s[8:9]
	;;#ASMEND
"""

PROTECTED = """
	v_lshl_add_u64 v[2:3], s[22:23], 0, v[2:3]
	s_mov_b32 m0, s10
	v_readfirstlane_b32 s9, v3
	v_readfirstlane_b32 s8, v2
	;;#ASMSTART
	s_nop 4
	global_load_lds_dwordx4 v104, s[8:9]
	;;#ASMEND
	s_add_i32 m0, s10, 0x400
	;;#ASMSTART
	s_nop 0
	global_load_lds_dwordx4 v102, s[8:9]
	;;#ASMEND
"""

VGPR_ADDRESS = """
	v_readfirstlane_b32 s9, v3
	s_mov_b32 m0, s2
	v_mov_b32_e32 v5, v9
	global_load_lds_dwordx4 v[4:5], off
"""


def test_stale_sgpr_base_is_flagged():
    found = asm_hazards.check(STALE_BASE)
    kinds = [k for k, _, _ in found]
    # s8 and s9, for both loads: the second is still within five wait states
    assert kinds.count("valu-sgpr") == 4
    assert kinds.count("m0") == 1                 # the second load
    assert {p.split()[1].rstrip(",") for k, p, _ in found if k == "valu-sgpr"} == {"s8", "s9"}


def test_wait_states_clear_both_hazards():
    assert asm_hazards.check(PROTECTED) == []


def test_vgpr_addressed_load_only_needs_m0_spacing():
    assert asm_hazards.check(VGPR_ADDRESS) == []
    assert [k for k, _, _ in asm_hazards.check(VGPR_ADDRESS.replace(
        "\tv_mov_b32_e32 v5, v9\n", ""))] == ["m0"]


# The cache writer's device-scope stores, as the compiler lays out an asm block:
# a 16-byte store must be followed in its block by s_nop 1 or more (two wait
# states before a VALU write of its data VGPRs).
STORE_PROTECTED = """
	v_cvt_pk_fp8_f32 v13, v10, v11
	;;#ASMSTART
	global_store_dwordx4 v[26:27], v[10:13], off sc1
	s_nop 1
	;;#ASMEND
	v_mov_b32_e32 v10, 0
"""


def test_asm_store_with_wait_states_is_clean():
    assert asm_hazards.check_stores(STORE_PROTECTED) == []


def test_asm_store_without_wait_states_is_flagged():
    bare = STORE_PROTECTED.replace("\ts_nop 1\n", "")
    assert asm_hazards.check_stores(bare) == ["global_store_dwordx4 v[26:27], v[10:13], off sc1"]
    one = STORE_PROTECTED.replace("s_nop 1", "s_nop 0")       # one wait state only
    assert len(asm_hazards.check_stores(one)) == 1


def test_narrow_and_compiler_stores_are_not_asm_hazards():
    narrow = STORE_PROTECTED.replace("dwordx4 v[26:27], v[10:13]", "dwordx2 v[26:27], v[10:11]")
    assert asm_hazards.check_stores(narrow.replace("\ts_nop 1\n", "")) == []
    outside = "\tglobal_store_dwordx4 v[26:27], v[10:13], off\n\tv_mov_b32_e32 v10, 0\n"
    assert asm_hazards.check_stores(outside) == []
