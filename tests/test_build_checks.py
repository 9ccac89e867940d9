"""The build's checks on the gfx950 assembly (no GPU needed): matrix-core accumulations
with partly overlapping destination / accumulator registers, or fed by a matrix-core
instruction of another shape just before, fail the build."""
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


def test_mixed_shape_chain_detected():
    bad = ("  v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]\n"
           "  v_accvgpr_read_b32 v1, a4\n"
           "  v_mfma_f32_16x16x16_f16 a[0:3], v[2:3], v[4:5], a[0:3]\n")
    assert len(mfma_mixed_chains(bad)) == 1
    assert mfma_mixed_chains(CHAIN_OK) == []
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
        assert mfma_partial_overlaps(text) == [], fn
        assert mfma_mixed_chains(text) == [], fn
