"""Host-side checks of the build step (no GPU): the scan that rejects matrix-core instructions
whose destination registers overlap an A/B source."""
from causal_head_attention_gqa_amd.build import mfma_overlaps


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
