"""The inline-asm MFMA hazard check (sub_byte_mixed_amd/asm_hazards.py).

Snippets pin what it must flag and what it must pass; the built device
assembly of the kernels that issue asm MFMAs is checked when present (the
build itself refuses to link on a violation)."""
import os

import pytest

from sub_byte_mixed_amd import asm_hazards as H
from sub_byte_mixed_amd import build as B


def _kernel(body: str) -> str:
    return "_Zk_probe_kernel:\n" + body + "\n\ts_endpgm\n.Lfunc_end0:\n"


def _mfma(dst: str, a: str = "v[0:3]", b: str = "v[4:7]") -> str:
    return f";;#ASMSTART\n\tv_mfma_f32_16x16x32_f16 {dst}, {a}, {b}, {dst}\n;;#ASMEND"


def _violations(body: str):
    (n, bad), = H.check_asm(_kernel(body), "_probe_kernel").values()
    return n, bad


def test_flags_agpr_move_between_asm_mfmas():
    # the compiler-placed accumulator rotation that once corrupted one
    # accumulator: a move into a4 right before an MFMA that reads a[4:7]
    n, bad = _violations("\n".join([_mfma("a[0:3]"), "\tv_accvgpr_mov_b32 a4, a0", _mfma("a[4:7]")]))
    assert n == 2
    assert any("writes an operand" in b for b in bad)
    assert any("touches the result" in b for b in bad)


def test_guarded_read_passes():
    body = "\n".join([_mfma("a[0:3]"), "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7", "\tv_accvgpr_read_b32 v8, a0"])
    assert _violations(body)[1] == []


def test_short_guard_is_flagged():
    body = "\n".join([_mfma("a[0:3]"), "\ts_nop 7\n\ts_nop 7", "\tv_accvgpr_read_b32 v8, a2"])
    assert _violations(body)[1]


def test_in_place_accumulation_chain_passes():
    body = "\n".join([_mfma("a[0:3]"), _mfma("a[4:7]"), _mfma("a[0:3]"), _mfma("a[4:7]")])
    assert _violations(body)[1] == []


def test_valu_write_right_before_operand_read_is_flagged():
    body = "\n".join(["\tv_pk_mul_f16 v2, v9, v10", _mfma("a[0:3]")])
    assert _violations(body)[1]
    spaced = "\n".join(["\tv_pk_mul_f16 v2, v9, v10", "\ts_nop 3", _mfma("a[0:3]")])
    assert _violations(spaced)[1] == []


def test_scale_operand_write_is_flagged():
    # a scaled MFMA reads its two E8M0 scale registers as well
    mx = (";;#ASMSTART\n\tv_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[0:3], v[4:7], a[0:3], v8, v9 "
          "op_sel_hi:[0,0,0] cbsz:4 blgp:4\n;;#ASMEND")
    assert _violations("\n".join(["\tv_lshrrev_b32_e32 v9, v10, v11", mx]))[1]
    assert _violations("\n".join(["\tv_lshrrev_b32_e32 v9, v10, v11", "\ts_nop 3", mx]))[1] == []


def test_hazard_on_one_branch_path_is_flagged():
    # the straight-line order is safe; the taken branch skips the guard
    body = "\n".join([
        _mfma("a[0:3]"),
        "\ts_cbranch_scc1 .LBB0_2",
        "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7",
        ".LBB0_2:",
        "\tv_accvgpr_read_b32 v8, a1",
    ])
    assert _violations(body)[1]


def test_flat_memory_access_is_flagged():
    # a flat store also counts in lgkmcnt, which the K loop's barriers wait on
    body = "\n".join([_mfma("a[0:3]"), "\tflat_store_dwordx4 v[34:35], v[0:3] offset:64"])
    assert any("flat memory access" in b for b in _violations(body)[1])
    body = "\n".join([_mfma("a[0:3]"), "\tglobal_store_dwordx4 v[34:35], v[0:3], off offset:64"])
    assert _violations(body)[1] == []


def test_compiler_selected_mfma_is_not_checked():
    # outside an asm region the compiler inserts the wait states itself
    body = "\tv_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]\n\tv_accvgpr_read_b32 v8, a0"
    n, bad = _violations(body)
    assert n == 0 and bad == []


def test_built_device_assembly():
    for src, kernels in B.ASM_MFMA_KERNELS.items():
        path = os.path.join(B.BUILD_DIR, os.path.splitext(src)[0] + ".device.s")
        if not os.path.exists(path):
            pytest.skip("no device assembly built here")
        B.check_asm_mfma(path, kernels)
