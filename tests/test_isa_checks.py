"""Checks of the compiled gfx950 kernels (CPU): the split-state scan's untracked
register loads of x are never overwritten or reused before their wait, on any
path; no direct-to-LDS load directly follows a write of M0; and no vector
memory instruction reads an SGPR that a VALU instruction wrote fewer than five
wait states before (inline assembly is not padded by the compiler)."""
import os
import shutil

import pytest

from isa_check import (HIPCC, kernel_asm, m0_lds_dma_hazards, untracked_load_violations,
                       valu_sgpr_vmem_hazards)

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def test_split_scan_untracked_x_loads():
    bad, count = untracked_load_violations(kernel_asm("ssd_scan_split_bf16.hip"))
    assert count >= 6, f"expected the prologue and per-step x loads, found {count}"
    assert not bad, "untracked load registers touched before their wait: " + "; ".join(
        f"load at line {ln}: {why}" for ln, why in bad[:5])


def test_checker_flags_a_reused_register():
    """A planted reuse: the destination is overwritten before any wait. Loads
    the compiler emits itself (outside inline assembly) are not counted."""
    text = "\n".join([
        "\t;;#ASMSTART", "\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen offset:0", "\t;;#ASMEND",
        "\tv_mov_b32_e32 v5, 0",
        "\ts_waitcnt vmcnt(0)",
        "\ts_endpgm"])
    bad, count = untracked_load_violations(text)
    assert count == 1 and len(bad) == 1
    ok = "\n".join([
        "\t;;#ASMSTART", "\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen offset:0", "\t;;#ASMEND",
        "\tbuffer_load_dwordx4 v[8:11], v1, s[0:3], 0 offen offset:0",
        "\ts_cbranch_scc1 .LBB0_2",
        "\ts_waitcnt vmcnt(0)",
        "\tv_mov_b32_e32 v5, 0",
        ".LBB0_2:",
        "\tds_write_b128 v9, v[4:7]",
        "\tv_mov_b32_e32 v9, v8",
        "\ts_endpgm"])
    assert untracked_load_violations(ok) == ([], 1)


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_bf16.hip", "ssd_scan_f32.hip"])
def test_m0_written_a_wait_state_before_lds_dma(src):
    bad, count = m0_lds_dma_hazards(kernel_asm(src))
    assert count > 0, "no direct-to-LDS loads found"
    assert not bad, f"{len(bad)} of {count} LDS-DMA loads right after an M0 write, e.g. line {bad[0][0]}"


def test_m0_checker_flags_a_planted_hazard():
    text = "\n".join(["\ts_mov_b32 m0, s4", "\tbuffer_load_dword v1, s[0:3], 0 offen lds",
                      "\ts_add_u32 m0, s5, 0x400", "\ts_nop 0",
                      "\tbuffer_load_dwordx4 v2, s[0:3], 0 offen lds"])
    bad, count = m0_lds_dma_hazards(text)
    assert count == 2 and [b[0] for b in bad] == [2]


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_bf16.hip", "ssd_scan_f32.hip",
                                 "ssd_decode.hip", "ssd_meta.hip"])
def test_valu_sgpr_write_five_wait_states_before_vmem(src):
    bad = valu_sgpr_vmem_hazards(kernel_asm(src))
    assert not bad, (f"{len(bad)} vector memory reads of a VALU-written SGPR too soon, e.g. line "
                     f"{bad[0][0]}: {bad[0][1]} after {bad[0][2]} ({bad[0][3]} wait states)")


def test_valu_sgpr_checker_flags_a_planted_hazard():
    text = "\n".join(["\tv_readfirstlane_b32 s68, v32", "\ts_and_b32 s69, s24, 0xffff",
                      "\ts_mov_b32 m0, s12", "\ts_nop 0",
                      "\tbuffer_load_dwordx4 v65, s[68:71], 0 offen lds",
                      "\tv_readfirstlane_b32 s70, v3", "\ts_nop 4",
                      "\tbuffer_load_dwordx4 v66, s[68:71], 0 offen lds"])
    bad = valu_sgpr_vmem_hazards(text)
    assert [b[0] for b in bad] == [5]
