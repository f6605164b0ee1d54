"""The split-state scan's untracked register loads of x are never overwritten
or reused before their wait, on any path of the compiled gfx950 code (CPU)."""
import os
import shutil

import pytest

from isa_check import CSRC, HIPCC, compile_asm, untracked_load_violations

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def test_split_scan_untracked_x_loads(tmp_path):
    asm = compile_asm(os.path.join(CSRC, "ssd_scan_split_bf16.hip"), str(tmp_path / "split.s"))
    bad, count = untracked_load_violations(open(asm).read())
    assert count >= 6, f"expected the prologue and per-step x loads, found {count}"
    assert not bad, "untracked load registers touched before their wait: " + "; ".join(
        f"load at line {ln}: {why}" for ln, why in bad[:5])


def test_checker_flags_a_reused_register():
    """A planted reuse: the destination is overwritten before any wait."""
    text = "\n".join([
        "\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen offset:0",
        "\tv_mov_b32_e32 v5, 0",
        "\ts_waitcnt vmcnt(0)",
        "\ts_endpgm"])
    bad, count = untracked_load_violations(text)
    assert count == 1 and len(bad) == 1
    ok = "\n".join([
        "\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen offset:0",
        "\ts_cbranch_scc1 .LBB0_2",
        "\ts_waitcnt vmcnt(0)",
        "\tv_mov_b32_e32 v5, 0",
        ".LBB0_2:",
        "\tds_write_b128 v9, v[4:7]",
        "\ts_endpgm"])
    assert untracked_load_violations(ok) == ([], 1)
