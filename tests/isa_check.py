"""Checks of compiled gfx950 code for the split-state scan (CPU only).

The scan loads x into registers with inline-assembly buffer loads that the
compiler does not track: it takes their destination registers as written at
once, waits for them only through the kernel's own explicit vmcnt waits, and
may hand a register it believes dead to another value while the load is still
in flight (the late load then overwrites that value). The invariant checked
here on the compiled code: on every control-flow path from such a load, the
first instruction that touches its destination registers is the store of
those registers into their LDS stage (which the kernel places after the wait
that covers the load), unless an `s_waitcnt vmcnt(0)` comes first.
"""
import functools
import os
import re
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_cu_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_asm(src, out, defines=()):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}",
           *[f"-D{d}" for d in defines], "--cuda-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


@functools.lru_cache(maxsize=None)
def kernel_asm(src):
    """Assembly text of one kernel source of the library, compiled once per session."""
    out = os.path.join(tempfile.mkdtemp(prefix="isa_"), os.path.basename(src) + ".s")
    compile_asm(os.path.join(CSRC, src), out)
    with open(out) as f:
        return f.read()


def _vregs(line):
    line = line.split(";")[0]
    out = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", line):
        out |= set(range(int(a), int(b) + 1))
    out |= {int(a) for a in re.findall(r"\bv(\d+)\b", line)}
    return out


def untracked_load_violations(asm_text):
    """(load line, path description) for every path that touches an untracked
    load's registers before its stage store or a vmcnt(0) wait; and the number
    of untracked loads found (register loads inside inline-assembly blocks)."""
    lines = asm_text.split("\n")
    labels = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = i
    bad, count = [], 0
    in_asm = False
    for i, l in enumerate(lines):
        s = l.strip()
        # only loads written in inline assembly (the compiler tracks its own)
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        if not (in_asm and s.startswith("buffer_load_dwordx4") and " lds" not in s and " offen" in s):
            continue
        m = re.search(r"v\[(\d+):(\d+)\]", s)
        a, b = int(m.group(1)), int(m.group(2))
        dst, tag = set(range(a, b + 1)), f"v[{a}:{b}]"
        count += 1
        stack, seen = [i + 1], set()
        while stack:
            j = stack.pop()
            while j < len(lines):
                if j in seen:
                    break
                seen.add(j)
                t = lines[j].strip()
                j += 1
                if not t or t.startswith(";") or t.startswith("."):
                    continue
                if t.startswith("s_endpgm"):
                    break
                if t.startswith("s_waitcnt") and "vmcnt(0)" in t:
                    break
                if t.startswith("ds_write_b128") and tag in t:
                    break
                if _vregs(t) & dst:
                    bad.append((i + 1, f"line {j}: {t}"))
                    break
                if t.startswith("s_branch"):
                    j = labels[t.split()[-1]]
                elif t.startswith("s_cbranch"):
                    stack.append(labels[t.split()[-1]])
    return bad, count


def m0_lds_dma_hazards(asm_text):
    """Direct-to-LDS loads (`... lds`) whose previous instruction writes M0.

    gfx9 parts need one wait state between a scalar write of M0 and an LDS-DMA
    load that reads it; without it the load may use the previous M0 (its data
    then lands on the previous block's LDS address). Returns (line, text) of
    each offending load and the number of LDS-DMA loads seen."""
    prev, bad, count = None, [], 0
    for i, l in enumerate(asm_text.split("\n")):
        t = l.strip()
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        if t.startswith("buffer_load") and t.endswith(" lds"):
            count += 1
            if prev is not None and re.match(r"^s_\w+\s+m0\b", prev):
                bad.append((i + 1, t))
        prev = t
    return bad, count


def _sregs(text):
    out = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", text):
        out |= set(range(int(a), int(b) + 1))
    out |= {int(a) for a in re.findall(r"\bs(\d+)\b", text)}
    return out


def valu_sgpr_vmem_hazards(asm_text, need=5):
    """Vector memory instructions that read an SGPR written by a VALU
    instruction (v_readfirstlane, v_readlane, v_cmp ... into SGPRs) fewer than
    `need` wait states earlier (gfx9 needs 5; each instruction in between is
    one wait state, s_nop N is N + 1). Straight-line view of the code (a branch
    target is treated as following the instruction above it)."""
    ins = []
    for i, l in enumerate(asm_text.split("\n")):
        t = l.strip()
        if t and not t.startswith(";") and not t.startswith(".") and not t.endswith(":"):
            ins.append((i + 1, t))
    bad = []
    for k, (ln, t) in enumerate(ins):
        if not (t.startswith("buffer_") or t.startswith("global_")):
            continue
        rd = _sregs(t.split(None, 1)[1]) if " " in t else set()
        ws = 0
        for j in range(k - 1, -1, -1):
            p = ins[j][1]
            if p.startswith("v_") and " " in p:
                dst = p.split(None, 1)[1].split(",")[0]
                if _sregs(dst) & rd:
                    bad.append((ln, t, ins[j][1], ws))
                    break
            ws += int(p.split()[1]) + 1 if p.startswith("s_nop") else 1
            if ws >= need:
                break
    return bad
