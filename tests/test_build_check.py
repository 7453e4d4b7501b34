"""The build's check of matrix instructions (_build.check_mfma_fences) on
small assembly listings: the control-flow walk accepts kernels whose
accumulators are touched only after the drain (or, for the builtin
instruction, inside the block of the instruction), and rejects an access
between hand-tied instructions, an access in a merge block before the drain,
and a zero fill not followed by wait states."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location(
    "mfl_build", os.path.join(ROOT, "mma_fragment_layouts_tn_amd", "_build.py"))
B = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(B)

T16 = "v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]"
T32 = "v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]"
DRAIN = ("s_nop 7", "s_nop 7", "s_nop 7")


def _kernel(*body):
    return "\n".join(["_Zkernel:", *body, "s_endpgm", ".Lfunc_end0:"])


def test_accepts_a_clean_tied_kernel():
    k = _kernel("v_accvgpr_write_b32 a0, 0", "s_nop 4", T16, "ds_read_b128 v[8:11], v1", T16,
                *DRAIN, "v_accvgpr_read_b32 v2, a0")
    assert B.check_mfma_fences(k, "good") == 1


@pytest.mark.parametrize("body,why", [
    (("s_nop 4", T16, "v_accvgpr_read_b32 v2, a0", T16, *DRAIN), "in flight"),
    (("s_nop 4", T16, "v_accvgpr_mov_b32 a4, a0", T16, *DRAIN), "in flight"),
    (("s_nop 4", T16, "v_accvgpr_read_b32 v2, a0", *DRAIN), "in flight"),
    (("s_nop 4", T16, "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v2, a0"), "in flight"),
    (("v_accvgpr_write_b32 a0, 0", T16, *DRAIN), "zero fill"),
])
def test_rejects_tied(body, why):
    with pytest.raises(RuntimeError, match=why):
        B.check_mfma_fences(_kernel(*body), "bad")


def test_tied_access_on_another_path_is_found():
    """The instruction in a conditional block, the read in the block after
    the join: found through the control-flow graph, not the listing order."""
    k = _kernel("s_nop 4", "s_cbranch_scc1 .LBB0_2", ".LBB0_1:", T16, "s_branch .LBB0_3",
                ".LBB0_2:", "s_nop 0", ".LBB0_3:", "v_accvgpr_read_b32 v2, a0", *DRAIN)
    with pytest.raises(RuntimeError, match="in flight"):
        B.check_mfma_fences(k, "bad")


def test_builtin_kernels_checked_at_merge_blocks_only():
    inside = _kernel("s_nop 4", T32, "v_accvgpr_read_b32 v2, a20", T32, *DRAIN)
    assert B.check_mfma_fences(inside, "builtin", tied=False) == 1
    single = _kernel("s_nop 4", T32, "s_branch .LBB0_1", ".LBB0_1:", "v_accvgpr_read_b32 v2, a3",
                     *DRAIN)
    assert B.check_mfma_fences(single, "builtin", tied=False) == 1
    merge = _kernel("s_nop 4", "s_cbranch_scc1 .LBB0_2", ".LBB0_1:", T32, ".LBB0_2:",
                    "v_accvgpr_read_b32 v2, a3", *DRAIN)
    with pytest.raises(RuntimeError, match="in flight"):
        B.check_mfma_fences(merge, "builtin", tied=False)
    drained = _kernel("s_nop 4", "s_cbranch_scc1 .LBB0_2", ".LBB0_1:", T32, ".LBB0_2:", *DRAIN,
                      "v_accvgpr_read_b32 v2, a3")
    assert B.check_mfma_fences(drained, "builtin", tied=False) == 1


def test_kernel_kind_is_decided_by_its_instructions():
    """A kernel with only builtin instructions gets the builtin rules (an
    access inside the instruction's block is the compiler's to fence); with
    the tied rules forced it has no tied instruction and is not counted."""
    k = _kernel("s_nop 4", T32, "v_accvgpr_read_b32 v2, a3", T32)
    assert B.check_mfma_fences(k, "auto") == 1
    assert B.check_mfma_fences(k, "tied", tied=True) == 0
    with pytest.raises(RuntimeError, match="in flight"):
        B.check_mfma_fences(_kernel("s_nop 4", T16, "v_accvgpr_read_b32 v2, a3", T16), "auto")
