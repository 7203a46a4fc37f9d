"""The build's check on MFMAs written as inline asm: the compiler inserts no
wait states after them, so the build scans the device assembly for any access
to an MFMA's destination registers before 18 wait states have passed.  These
pin the scanner on hand-written assembly and check that it covers the sources
that need it."""
import os

from extreme_bit_quantized_amd import build as B

MF = "v_mfma_i32_16x16x64_i8 a[112:115], v[48:51], v[68:71], a[112:115]"


def _fn(*body):
    return "\n".join(["_Zkernel:"] + ["\t" + b for b in body] + ["\ts_endpgm"])


def test_read_right_after_mfma_flagged():
    bad = B.mfma_result_hazards(_fn(MF, "s_nop 0", "v_accvgpr_read_b32 v96, a112"))
    assert len(bad) == 1 and bad[0][1] == 2 and "a112" in bad[0][2]


def test_read_after_wait_states_passes():
    asm = _fn(MF, "s_nop 7", "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v96, a112",
              "v_accvgpr_read_b32 v97, a115")
    assert B.mfma_result_hazards(asm) == []


def test_every_register_of_the_destination_checked():
    asm = _fn(MF, "s_nop 7", "s_nop 6", "v_accvgpr_read_b32 v96, a112", "v_accvgpr_read_b32 v97, a115")
    bad = B.mfma_result_hazards(asm)
    assert [b[2].split()[-1] for b in bad] == ["a112", "a115"]


def test_accumulation_chain_and_other_registers_pass():
    asm = _fn(MF, MF, "v_accvgpr_read_b32 v1, a116", "ds_read_b128 v[48:51], v7",
              "s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v2, a113")
    assert B.mfma_result_hazards(asm) == []


def test_vgpr_destination_and_operand_use_flagged():
    mf = "v_mfma_i32_32x32x32_i8 v[0:15], v[16:19], v[20:23], v[0:15]"
    bad = B.mfma_result_hazards(_fn(mf, "v_cvt_f32_i32_e32 v30, v3"))
    assert len(bad) == 1 and bad[0][1] == 1
    # an MFMA reading another MFMA's fresh result as an A/B operand
    bad = B.mfma_result_hazards(_fn(mf, "v_mfma_i32_32x32x32_i8 v[32:47], v[0:3], v[20:23], v[32:47]"))
    assert len(bad) == 1


def test_new_function_resets():
    asm = _fn(MF) + "\n" + "_Zother:\n\tv_accvgpr_read_b32 v96, a112\n"
    assert B.mfma_result_hazards(asm) == []


def test_sources_with_asm_mfma_are_checked():
    csrc = os.path.join(os.path.dirname(B.__file__), "csrc")
    checked = []
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".hip"):
            with open(os.path.join(csrc, name)) as f:
                if B._ASM_MFMA.search(f.read()):
                    checked.append(name)
    assert "gemm_rs.hip" in checked and "gemm.hip" in checked
