"""The build's check on the gfx950 assembly (no GPU needed): a matrix-core accumulation fed
by a matrix-core instruction of another shape just before fails the build; a destination
that partly overlaps the accumulator input within a one-shape chain does not."""
import glob
import os

from gated_deltanet_chunked_02_amd.build import (BUILD, mfma_mixed_chains,
                                                 mfma_partial_overlaps)

CHAIN_OK = """
  v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]
  v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[14:17], a[0:3]
  v_mfma_f32_16x16x32_f16 a[4:7], v[10:13], v[14:17], a[0:3]
  v_mfma_f32_16x16x16_f16 a[8:11], v[2:3], v[4:5], 0
"""


def test_partial_overlap_detected():
    bad = "  v_mfma_f32_16x16x32_f16 a[2:5], v[54:57], v[14:17], a[4:7]\n"
    assert len(mfma_partial_overlaps(bad)) == 1
    assert mfma_partial_overlaps(CHAIN_OK) == []
    # different register files never overlap
    assert mfma_partial_overlaps("  v_mfma_f32_16x16x32_bf16 v[2:5], v[6:9], v[10:13], a[4:7]\n") == []


def test_mixed_shape_chain_with_partial_overlap_detected():
    # the pair that gave wrong sums: a 16x16x32 result in a[2:5] fed at once into a 16x16x16
    # accumulation, each destination shifted against its accumulator input
    bad = ("  v_mfma_f32_16x16x32_f16 a[2:5], v[54:57], v[14:17], a[4:7]\n"
           "  v_accvgpr_read_b32 v1, a0\n"
           "  v_mfma_f32_16x16x16_f16 a[4:7], v[38:39], v[26:27], a[2:5]\n")
    assert len(mfma_mixed_chains(bad)) == 1
    # a one-shape chain whose destinations shift against the inputs is accepted
    ok = ("  v_mfma_f32_16x16x32_bf16 v[128:131], v[190:193], v[90:93], v[128:131]\n"
          "  v_mfma_f32_16x16x32_bf16 v[134:137], v[202:205], v[90:93], v[132:135]\n"
          "  v_mfma_f32_16x16x32_bf16 v[130:133], v[186:189], v[98:101], v[128:131]\n"
          "  v_mfma_f32_16x16x32_bf16 v[134:137], v[210:213], v[98:101], v[134:137]\n")
    assert len(mfma_partial_overlaps(ok)) == 2
    assert mfma_mixed_chains(ok) == []


def test_mixed_shape_chain_detected():
    bad = ("  v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
           "  v_accvgpr_read_b32 v1, a4\n"
           "  v_mfma_f32_16x16x16_f16 a[0:3], v[2:3], v[4:5], a[0:3]\n")
    assert len(mfma_mixed_chains(bad)) == 1
    assert mfma_mixed_chains(CHAIN_OK) == []
    # an accumulator overwritten in between by the reader's own shape is not flagged
    over = ("  v_mfma_f32_16x16x16_f16 a[20:23], v[10:11], v[6:7], 0\n"
            "  v_mfma_f32_16x16x32_f16 a[20:23], v[40:43], v[14:17], 0\n"
            "  v_mfma_f32_16x16x32_f16 a[20:23], v[2:5], v[6:9], a[20:23]\n")
    assert mfma_mixed_chains(over) == []
    # ... and so is one rewritten by another instruction in between
    moved = ("  v_mfma_f32_16x16x32_bf16 a[16:19], v[30:33], v[10:13], 0\n"
             "  v_accvgpr_write_b32 a16, v69\n"
             "  v_accvgpr_write_b32 a17, v74\n"
             "  v_accvgpr_write_b32 a18, v75\n"
             "  v_accvgpr_write_b32 a19, v76\n"
             "  v_mfma_f32_16x16x32_f16 a[16:19], v[88:91], v[6:9], a[16:19]\n")
    assert mfma_mixed_chains(moved) == []
    # a store only reads its first operand
    kept = ("  v_mfma_f32_16x16x32_bf16 v[16:19], v[30:33], v[10:13], 0\n"
            "  ds_write_b128 v16, v[20:23]\n"
            "  v_mfma_f32_16x16x32_f16 v[16:19], v[88:91], v[6:9], v[16:19]\n")
    assert len(mfma_mixed_chains(kept)) == 1
    # a partly overlapping input is checked register by register
    part = ("  v_mfma_f32_16x16x16_f16 a[4:7], v[10:11], v[6:7], 0\n"
            "  v_mfma_f32_16x16x32_f16 a[0:3], v[40:43], v[14:17], 0\n"
            "  v_mfma_f32_16x16x32_f16 a[8:11], v[2:5], v[6:9], a[2:5]\n")
    assert len(mfma_mixed_chains(part)) == 1
    # far enough apart (beyond the window) is not flagged
    far = bad.replace("  v_accvgpr_read_b32 v1, a4\n", "  v_nop\n" * 20)
    assert mfma_mixed_chains(far) == []


def test_built_assembly_is_clean():
    files = glob.glob(os.path.join(BUILD, "*.gfx950.s"))
    if not files:
        import pytest
        pytest.skip("no build output")
    for fn in files:
        text = open(fn).read()
        assert mfma_mixed_chains(text) == [], fn


def test_no_kernel_uses_scratch():
    """Every kernel of the build keeps its values in registers and LDS: the code-object
    metadata gives each kernel's private (scratch) bytes per lane, which must be zero (a
    spill or a stack array would put per-lane memory traffic into the hot loops)."""
    import re
    files = glob.glob(os.path.join(BUILD, "*.gfx950.s"))
    if not files:
        import pytest
        pytest.skip("no build output")
    seen = 0
    for fn in files:
        text = open(fn).read()
        for blk in re.findall(r"- \.agpr_count:.*?\.vgpr_spill_count:\s*\d+", text, re.S):
            name = re.search(r"\.name:\s+(\S+)", blk).group(1)
            private = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk).group(1))
            assert private == 0, (os.path.basename(fn), name, private)
            seen += 1
    assert seen > 20
