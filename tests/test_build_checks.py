"""The assembly checks of build.py, on hand-written snippets (no GPU): each
catches a planted mistake and passes the same snippet without it."""
import pytest

from mla_tree_verify_latent_amd import build as B

KERNEL = "probe_kernelILi3E"


def _asm(lines):
    return f"_ZN4test{KERNEL}Ev:\n" + "".join(f"\t{l}\n" for l in lines) + "\ts_endpgm\n"


QK = "v_mfma_f32_16x16x32_bf16 v[4:7], v[128:131], a[72:75], v[4:7]"


def test_write_right_before_an_asm_mfma_source():
    for bad in (["v_accvgpr_write_b32 a75, v154", QK],          # B operand (AGPR)
                ["v_mov_b32 v129, v3", "s_waitcnt lgkmcnt(0)", QK],  # A operand (VGPR), a wait issues nothing
                ["v_accvgpr_mov_b32 a72, a90", "s_nop 0", QK]):  # one wait state is not two
        with pytest.raises(RuntimeError):
            B.check_mfma_hazards(_asm(bad), KERNEL)
    B.check_mfma_hazards(_asm(["v_accvgpr_write_b32 a75, v154", "s_nop 1", QK]), KERNEL)
    B.check_mfma_hazards(_asm(["v_mov_b32 v200, v3", QK]), KERNEL)


def test_query_agprs_stay_put_between_qk_mfmas():
    bad = [QK, "v_accvgpr_write_b32 a73, v171", "s_nop 7", QK]
    with pytest.raises(RuntimeError):
        B.check_asm_b_operands_invariant(_asm(bad), KERNEL)
    B.check_asm_b_operands_invariant(_asm([QK, "v_accvgpr_write_b32 a80, v171", QK]), KERNEL)
    B.check_asm_b_operands_invariant(_asm(["v_accvgpr_write_b32 a73, v171", "s_nop 7", QK, QK]), KERNEL)


def test_asm_mfma_result_read_before_drain():
    for bad in ([QK, "v_add_f32_e32 v10, v5, v11", "s_nop 7"],
                [QK, "ds_write_b128 v2, v[4:7] offset:16", "s_nop 7"],
                [QK, QK, "v_mul_f32_e32 v10, 0x3f000000, v6", "s_nop 7"],
                [QK, "v_mfma_f32_16x16x32_bf16 v[8:11], v[128:131], a[76:79], 0", "v_add_f32_e32 v10, v5, v11",
                 "s_nop 7"]):
        with pytest.raises(RuntimeError):
            B.check_asm_mfma_result_reads(_asm(bad), KERNEL)
    B.check_asm_mfma_result_reads(_asm([QK, "s_nop 7", "v_add_f32_e32 v10, v5, v11"]), KERNEL)
    B.check_asm_mfma_result_reads(_asm([QK, "v_add_f32_e32 v10, v50, v11", "s_nop 7"]), KERNEL)
