"""Host-side checks of the build step (no GPU): the scans that reject matrix-core instructions
whose destination registers overlap an A/B source, and direct-to-LDS loads whose SGPR base
address was sign-extended from 32 bits."""
import glob
import os

from causal_head_attention_gqa_amd.build import BUILD, mfma_overlaps, sign_extended_lds_bases


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


def test_built_kernels_pass_both_scans():
    files = glob.glob(os.path.join(BUILD, "*.s"))
    if not files:
        import pytest
        pytest.skip("no generated assembly: run the build first")
    for f in files:
        text = open(f).read()
        assert mfma_overlaps(text) == [], f
        assert sign_extended_lds_bases(text) == [], f
