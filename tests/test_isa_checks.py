"""Checks of the compiled gfx950 kernels (CPU): every explicit stage wait of the
scan pipelines has, on every path, at least as many vector memory instructions
after the stage's last load as its vmcnt assumes; the split-state scan's
untracked register loads of x are never overwritten or reused before their
wait, on any path; no direct-to-LDS load directly follows a write of M0; and no
vector memory instruction reads an SGPR that a VALU instruction wrote fewer
than five wait states before (inline assembly is not padded by the compiler);
and no kernel spills to scratch memory (a register array indexed at run time
lands there, and its loads then wait behind the pipelines' vector memory)."""
import os
import shutil

import pytest

from isa_check import (HIPCC, kernel_asm, kernel_resources, m0_lds_dma_hazards, untracked_load_violations,
                       store_data_hazards, valu_sgpr_vmem_hazards, vmcnt_stage_violations)

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip"])
def test_split_scan_untracked_x_loads(src):
    bad, count = untracked_load_violations(kernel_asm(src))
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


def test_untracked_checker_follows_constant_flags():
    """Where the structurizer joins two wave-uniform branches through a flag
    that is a known constant, the branch it guards always goes one way: the
    other edge is not a path. A flag of -1 takes the fall-through instead."""
    def text(flag):
        return "\n".join([
            "\t;;#ASMSTART", "\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen offset:0", "\t;;#ASMEND",
            f"\ts_mov_b64 s[10:11], {flag}",
            "\ts_and_b64 vcc, exec, s[10:11]",
            "\ts_cbranch_vccz .LBB0_9",
            "\tv_mov_b32_e32 v5, 0",
            ".LBB0_9:",
            "\tds_write_b128 v9, v[4:7]",
            "\ts_endpgm"])
    assert untracked_load_violations(text(0)) == ([], 1)
    bad, count = untracked_load_violations(text(-1))
    assert count == 1 and len(bad) == 1


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_scan_bf16.hip",
                                 "ssd_scan_f32.hip"])
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


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_scan_bf16.hip",
                                 "ssd_scan_f32.hip", "ssd_decode.hip", "ssd_meta.hip"])
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


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_scan_bf16.hip",
                                 "ssd_scan_f32.hip"])
def test_stage_waits_cover_their_loads(src):
    """Each `s_waitcnt vmcnt(n)` that releases a pipeline stage sees at least
    n vector memory instructions after that stage's last load, on every path,
    in every compiled instance (placeholder stores the compiler merged or
    dropped would leave fewer)."""
    bad, counts = vmcnt_stage_violations(kernel_asm(src))
    pipelined = [f for f, (nl, nw) in counts.items() if nw > 0]
    assert pipelined, "no tagged stage waits found"
    assert all(counts[f][0] > 0 for f in pipelined), "tagged waits without tagged loads"
    assert not bad, f"{len(bad)} stage waits with too few instructions after the stage's loads, e.g. " + \
        "; ".join(f"{f[:48]}.. line {ln}: stage {k} waits vmcnt({n}) after {d}" for f, ln, k, n, d in bad[:3])


def _kernel(lines):
    return "\n".join(["_Z4testv:"] + ["\t" + l if not l.endswith(":") else l for l in lines] +
                     [".Lfunc_end0:"])


def test_vmcnt_checker_flags_merged_placeholder_stores():
    """Planted: two placeholder stores were expected after the stage's load,
    the compiler left one, and the wait still assumes two."""
    load = "buffer_load_dwordx4 v1, s[0:3], 0 offen lds ; ssd-stage 0"
    bad, _ = vmcnt_stage_violations(_kernel([
        load, "buffer_store_dwordx2 v[2:3], off, s[4:7], 0",
        "s_waitcnt vmcnt(2) ; ssd-wait 0 excl 0", "s_endpgm"]))
    assert [(b[2], b[3], b[4]) for b in bad] == [(0, 2, 1)]
    ok, _ = vmcnt_stage_violations(_kernel([
        load, "buffer_store_dwordx2 v[2:3], off, s[4:7], 0", "buffer_store_dwordx2 v[2:3], off, s[4:7], 0",
        "s_waitcnt vmcnt(2) ; ssd-wait 0 excl 0", "s_endpgm"]))
    assert ok == []


def test_vmcnt_checker_paths_exports_and_structurizer_edges():
    """A path that skips an instruction fails; export stores only count as
    the wait declares; a loop exit through s_cbranch_execnz with a full exec
    mask never falls through; a flag set to -1 selects its branch."""
    load = "buffer_load_dwordx4 v1, s[0:3], 0 offen lds ; ssd-stage 1"
    store = "buffer_store_dwordx2 v[2:3], off, s[4:7], 0"
    bad, _ = vmcnt_stage_violations(_kernel([
        load, "s_cbranch_scc1 .LBB0_2", store, ".LBB0_2:",
        "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0", "s_endpgm"]))
    assert len(bad) == 1
    export = "buffer_store_dwordx4 v[2:5], v6, s[4:7], 0 offen ; ssd-export"
    ok, _ = vmcnt_stage_violations(_kernel([load, store, export, "s_waitcnt vmcnt(2) ; ssd-wait 1 excl 1", "s_endpgm"]))
    assert ok == []
    bad, _ = vmcnt_stage_violations(_kernel([load, export, export, "s_waitcnt vmcnt(2) ; ssd-wait 1 excl 0", "s_endpgm"]))
    assert len(bad) == 1
    # a wait that releases two stages is checked for both
    load5 = "buffer_load_dwordx4 v1, s[0:3], 0 offen lds ; ssd-stage 5"
    bad, _ = vmcnt_stage_violations(_kernel([load5, store, load, store, "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0 ; ssd-wait 5 excl 0",
                                             "s_endpgm"]))
    assert bad == []
    bad, _ = vmcnt_stage_violations(_kernel([load, store, load5, "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0 ; ssd-wait 5 excl 0",
                                             "s_endpgm"]))
    assert [b[2] for b in bad] == [5]
    ok, _ = vmcnt_stage_violations(_kernel([
        load, "s_cbranch_execnz .LBB0_9",
        "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0", ".LBB0_9:", "s_endpgm"]))
    assert ok == []
    ok, _ = vmcnt_stage_violations(_kernel([
        load, "s_mov_b64 s[44:45], -1", "s_and_b64 vcc, exec, s[44:45]", "s_cbranch_vccnz .LBB0_9",
        "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0", ".LBB0_9:", "s_endpgm"]))
    assert ok == []
    bad, _ = vmcnt_stage_violations(_kernel([
        load, "s_and_saveexec_b64 s[2:3], vcc", "s_cbranch_execnz .LBB0_9",
        "s_waitcnt vmcnt(1) ; ssd-wait 1 excl 0", ".LBB0_9:", "s_endpgm"]))
    assert len(bad) == 1


@pytest.mark.parametrize("src", ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_scan_bf16.hip",
                                 "ssd_scan_f32.hip", "ssd_decode.hip", "ssd_meta.hip", "ssd_conv1d.hip"])
def test_wide_store_data_not_overwritten_at_once(src):
    bad, count = store_data_hazards(kernel_asm(src))
    assert not bad, (f"{len(bad)} of {count} wide stores have their data registers overwritten by the "
                     f"next instruction, e.g. line {bad[0][0]}: {bad[0][1]} then {bad[0][2]}")


def test_store_data_checker_flags_a_planted_hazard():
    text = "\n".join(["\tbuffer_store_dwordx4 v[2:5], v193, s[44:47], 0 offen",
                      "\tv_accvgpr_read_b32 v2, a20",
                      "\tbuffer_store_dwordx4 v[6:9], v193, s[44:47], 0 offen",
                      "\ts_nop 0",
                      "\tv_accvgpr_read_b32 v6, a20",
                      "\tbuffer_store_dwordx4 v[14:17], v193, s[44:47], 0 offen",
                      "\ts_nop 1",
                      "\tv_accvgpr_read_b32 v14, a20",
                      "\tglobal_store_dwordx4 v[0:1], v[10:13], off",
                      "\ts_add_u32 s0, s0, 1",
                      "\tv_mov_b32_e32 v11, 0"])
    bad, count = store_data_hazards(text)
    assert count == 4 and [b[0] for b in bad] == [1, 3, 9]


ALL_SOURCES = ["ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_scan_bf16.hip", "ssd_scan_f32.hip", "ssd_decode.hip",
               "ssd_conv1d.hip", "ssd_gdn.hip", "ssd_meta.hip"]


# The general kernel's bf16 instances for dstate 256 on one or two waves (headdim
# 16 or 32) hold 64 state floats per lane plus their fragments and spill
# registers to scratch; the stage-wait check above counts those memory
# instructions like any other. Every other kernel keeps everything in registers.
SPILL_ALLOWED = ("_ZN3ssd15ssd_scan_kernelItLi1ELi256EEEvNS_8ScanArgsEPKi",
                 "_ZN3ssd15ssd_scan_kernelItLi2ELi256EEEvNS_8ScanArgsEPKi")


@pytest.mark.parametrize("src", ALL_SOURCES)
def test_no_kernel_uses_scratch(src):
    res = kernel_resources(kernel_asm(src))
    assert res, f"no kernels found in {src}"
    spill = {k: v.get("private_segment_fixed_size") for k, v in res.items()
             if k not in SPILL_ALLOWED and
             (v.get("private_segment_fixed_size", 0) != 0 or v.get("vgpr_spill_count", 0) != 0)}
    assert not spill, f"kernels with scratch memory: {spill}"


def test_scratch_check_reads_the_metadata():
    text = "\n".join(["\t.amdgpu_metadata", "amdhsa.kernels:", "  - .agpr_count:     0",
                      "    .name:           k1", "    .private_segment_fixed_size: 144",
                      "    .vgpr_count:     64", "  - .agpr_count:     0", "    .name:           k2",
                      "    .private_segment_fixed_size: 0", "    .vgpr_count:     32"])
    res = kernel_resources(text)
    assert res["k1"]["private_segment_fixed_size"] == 144 and res["k2"]["private_segment_fixed_size"] == 0
