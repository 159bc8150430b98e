"""Host-side checks of the build step (no GPU): the scans of the generated gfx950 assembly that
reject matrix-core instructions whose destination registers overlap an A/B source, direct-to-LDS
loads whose SGPR base address was sign-extended from 32 bits, direct-to-LDS loads that read an
SGPR base a vector instruction wrote fewer than 5 wait states earlier, and direct-to-LDS loads
fewer wait states after an M0 write than the hazard needs (1 after a scalar, 5 after a vector
write). Each scan is pinned on the instruction sequence it exists for."""
import glob
import os

from causal_head_attention_gqa_amd.build import (BUILD, m0_lds_dma_hazards, mfma_overlaps, scan,
                                                 sign_extended_lds_bases, valu_sgpr_lds_hazards)


def test_overlap_scan_flags_destination_over_sources():
    asm = "\n".join([
        "\tv_mfma_f32_16x16x32_bf16 v[18:21], v[18:21], v[6:9], 0",        # dst == A
        "\tv_mfma_f32_32x32x16_bf16 v[34:49], v[40:43], v[74:77], 0",      # A inside dst
        "\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[12:15], v[10:13]",  # B overlaps dst
    ])
    assert len(mfma_overlaps(asm)) == 3


def test_overlap_scan_accepts_disjoint_and_accumulator_forms():
    asm = "\n".join([
        "\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]",   # dst == C is fine
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",       # different register files
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "\tv_add_f32 v1, v1, v2",
    ])
    assert mfma_overlaps(asm) == []


def test_lds_base_scan_flags_sign_extension():
    # the low word of the base, read with readfirstlane (a signed int), sign-extended into the pair
    asm = "\n".join([
        "\tv_readfirstlane_b32 s4, v134",
        "\tv_readfirstlane_b32 s7, v135",
        "\ts_mov_b32 s6, 0",
        "\ts_bfe_i64 s[4:5], s[4:5], 0x200000",
        "\ts_mov_b32 m0, s43",
        "\ts_or_b64 s[4:5], s[4:5], s[6:7]",
        "\t;;#ASMSTART",
        "\tglobal_load_lds_dwordx4 v150, s[4:5]",
    ])
    assert len(sign_extended_lds_bases(asm)) == 1


def test_lds_base_scan_accepts_zero_extended_pairs():
    asm = "\n".join([
        "\tv_readfirstlane_b32 s5, v133",
        "\tv_readfirstlane_b32 s4, v132",
        "\tglobal_load_lds_dwordx4 v147, s[4:5]",
        "\ts_bfe_i64 s[8:9], s[8:9], 0x200000",   # unrelated pair
        "\tglobal_load_lds_dwordx4 v148, s[4:5]",
    ])
    assert sign_extended_lds_bases(asm) == []


# the sequence of the second device fault of the 192-dim prefill variant: the SGPR base pair of an
# inline-assembly load written by v_readfirstlane right in front of it
_READFIRSTLANE_BASE = [
    "\tv_readfirstlane_b32 s5, v133",
    "\tv_readfirstlane_b32 s4, v132",
    "\ts_mov_b32 m0, s43",
    "\t;;#ASMSTART",
    "\ts_nop 0",
    "\tglobal_load_lds_dwordx4 v147, s[4:5]",
    "\t;;#ASMEND",
]


def test_sgpr_base_scan_flags_readfirstlane_right_before_the_load():
    assert len(valu_sgpr_lds_hazards("\n".join(_READFIRSTLANE_BASE))) == 1


def test_sgpr_base_scan_accepts_five_wait_states():
    asm = _READFIRSTLANE_BASE[:2] + ["\ts_nop 4"] + _READFIRSTLANE_BASE[2:]
    assert valu_sgpr_lds_hazards("\n".join(asm)) == []


def test_sgpr_base_scan_accepts_scalar_bases():
    asm = ["\ts_add_u32 s4, s10, s12", "\ts_addc_u32 s5, s11, 0"] + _READFIRSTLANE_BASE[2:]
    assert valu_sgpr_lds_hazards("\n".join(asm)) == []


def test_sgpr_base_scan_flags_a_label_inside_the_window():
    asm = ["\tv_readfirstlane_b32 s5, v133", "\tv_readfirstlane_b32 s4, v132", ".LBB0_7:"] + _READFIRSTLANE_BASE[2:]
    bad = valu_sgpr_lds_hazards("\n".join(asm))
    assert len(bad) == 1 and bad[0].startswith("label")


# the sequence the compiler emitted in front of every inline-assembly direct-to-LDS load before
# the s_nop 0 went into the asm: the M0 write directly before the load
_M0_THEN_LOAD = [
    "\tv_lshl_add_u64 v[10:11], v[16:17], 0, v[10:11]",
    "\ts_mov_b32 m0, s5",
    "\t;;#ASMSTART",
    "\tglobal_load_lds_dwordx4 v[10:11], off nt",
    "\t;;#ASMEND",
]


def test_m0_scan_flags_scalar_write_right_before_the_load():
    assert len(m0_lds_dma_hazards("\n".join(_M0_THEN_LOAD))) == 1
    other = ["\ts_add_i32 m0, s5, 0x800", "\t;;#ASMSTART", "\tglobal_load_lds_dwordx4 v[28:29], off nt"]
    assert len(m0_lds_dma_hazards("\n".join(other))) == 1


def test_m0_scan_accepts_one_wait_state():
    asm = _M0_THEN_LOAD[:3] + ["\ts_nop 0"] + _M0_THEN_LOAD[3:]
    assert m0_lds_dma_hazards("\n".join(asm)) == []
    # M0 written once for two loads: the second is further away still
    asm2 = asm + ["\t;;#ASMSTART", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v[12:13], off nt"]
    assert m0_lds_dma_hazards("\n".join(asm2)) == []


def test_m0_scan_flags_vector_write_within_five_wait_states():
    asm = ["\tv_readfirstlane_b32 m0, v7", "\ts_nop 2", "\tglobal_load_lds_dwordx4 v[2:3], off"]
    assert len(m0_lds_dma_hazards("\n".join(asm))) == 1
    asm = ["\tv_readfirstlane_b32 m0, v7", "\ts_nop 4", "\tglobal_load_lds_dwordx4 v[2:3], off"]
    assert m0_lds_dma_hazards("\n".join(asm)) == []


def test_m0_scan_flags_a_label_directly_before_the_load():
    asm = ["\ts_mov_b32 m0, s5", ".LBB3_2:", "\tglobal_load_lds_dwordx4 v[2:3], off"]
    bad = m0_lds_dma_hazards("\n".join(asm))
    assert len(bad) == 1 and bad[0].startswith("label")


def test_built_kernels_pass_every_scan():
    files = glob.glob(os.path.join(BUILD, "*.s"))
    if not files:
        import pytest
        pytest.skip("no generated assembly: run the build first")
    for f in files:
        for what, bad in scan(open(f).read()):
            assert bad == [], (f, what, bad[:3])
