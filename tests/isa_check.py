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
    from selective_state_space_cu_amd.build import SOURCE_FLAGS
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", *SOURCE_FLAGS.get(os.path.basename(src), []),
           f"-I{os.path.join(ROOT, 'include')}",
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


def _untracked_bodies(asm_text):
    """Per function: [(line, text, inside inline assembly)], labels as "name:"
    entries; a text with no function symbols is read as one function."""
    lines = asm_text.split("\n")
    have = any(re.match(r"^(_Z\w+):", l) for l in lines)
    out, name, body, in_asm = [], (None if have else "_text"), [], False
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):", l)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if l.startswith(".Lfunc_end"):
            out.append((name, body))
            name = None
            continue
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif re.match(r"^(\.LBB\d+_\d+):", t):
            body.append((i + 1, t.split(":")[0] + ":", False))
        elif t and not t.startswith(";") and not t.startswith("."):
            body.append((i + 1, t, in_asm))
    if name is not None and body:
        out.append((name, body))
    return out


def _split_blocks(body):
    """Basic blocks of a body of (line, text, ...) entries, and label -> block."""
    blocks, cur, label_of = [], [], {}
    for e in body:
        t = e[1]
        if t.endswith(":"):
            if cur:
                blocks.append(cur)
            cur = []
            label_of[t[:-1]] = len(blocks)
            continue
        cur.append(e)
        if t.startswith("s_branch") or t.startswith("s_cbranch") or t.startswith("s_endpgm"):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    return blocks, label_of


def _ckey(st):
    f, sv, c, v = st
    return (f, sv, tuple(sorted(c.items())), v)


def untracked_load_violations(asm_text):
    """(load line, path description) for every path that touches an untracked
    load's registers before its stage store or a vmcnt(0) wait; and the number
    of untracked loads found (register loads inside inline-assembly blocks).

    Paths follow the control-flow graph with the same scalar control state as
    the stage-wait check (exec known full, SGPR flags known 0 or -1, vcc known
    zero / non-zero), so edges that no wave can take -- the fall-through of a
    branch on a constant flag that the structurizer emits where two
    wave-uniform branches of a kernel join, or a loop exit through
    s_cbranch_execnz with a full mask -- are not followed."""
    bad, count = [], 0
    for _, body in _untracked_bodies(asm_text):
        blocks, label_of = _split_blocks(body)
        if not blocks:
            continue
        # control states reaching each block from the entry
        st0 = (True, frozenset(), {}, None)
        states = [dict() for _ in blocks]
        states[0][_ckey(st0)] = st0
        work = [(0, st0)]
        while work:
            bi, st = work.pop()
            for e in blocks[bi]:
                st = _exec_step(e[1], st)
            for sb in _edges(blocks[bi][-1][1], bi, len(blocks), label_of, st):
                k = _ckey(st)
                if k not in states[sb]:
                    states[sb][k] = st
                    work.append((sb, st))
        for bi, blk in enumerate(blocks):
            for k, (ln, t, in_asm) in enumerate(blk):
                if not (in_asm and t.startswith("buffer_load_dwordx4") and " lds" not in t and " offen" in t):
                    continue
                m = re.search(r"v\[(\d+):(\d+)\]", t)
                a, b = int(m.group(1)), int(m.group(2))
                dst, tag = set(range(a, b + 1)), f"v[{a}:{b}]"
                count += 1
                seen, stack = set(), []
                for st in states[bi].values():
                    for e in blk[:k + 1]:
                        st = _exec_step(e[1], st)
                    stack.append((bi, k + 1, st))
                done = False
                while stack and not done:
                    cb, ci, st = stack.pop()
                    key = (cb, ci, _ckey(st))
                    if key in seen:
                        continue
                    seen.add(key)
                    stopped = False
                    for (ln2, t2, _) in blocks[cb][ci:]:
                        if t2.startswith("s_endpgm"):
                            stopped = True
                            break
                        if t2.startswith("s_waitcnt") and _vmcnt_of(t2) == 0:
                            stopped = True
                            break
                        if t2.startswith("ds_write_b128") and tag in t2:
                            stopped = True
                            break
                        if _vregs(t2) & dst:
                            bad.append((ln, f"line {ln2}: {t2}"))
                            stopped = done = True
                            break
                        st = _exec_step(t2, st)
                    if stopped:
                        continue
                    for sb in _edges(blocks[cb][-1][1], cb, len(blocks), label_of, st):
                        stack.append((sb, 0, st))
    return bad, count


def m0_lds_dma_hazards(asm_text):
    """Direct-to-LDS loads (`... lds`) whose previous instruction writes M0.

    gfx9 parts need one wait state between a scalar write of M0 and an LDS-DMA
    load that reads it; without it the load may use the previous M0 (its data
    then lands on the previous block's LDS address). Returns (line, text) of
    each offending load and the number of LDS-DMA loads seen."""
    prev, bad, count = None, [], 0
    for i, l in enumerate(asm_text.split("\n")):
        t = l.split(";")[0].strip() if not l.strip().startswith(";") else l.strip()
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


_VMEM = re.compile(r"^(buffer_(load|store|atomic)|global_(load|store|atomic)|flat_(load|store|atomic)|scratch_)")
_INF = 64   # more than any vmcnt immediate (6 bits): "at least 64" behaves as "none outstanding"


def _functions(asm_text):
    """(name, [(line number, instruction text)]) per function of an assembly file."""
    out, name, body = [], None, []
    for i, l in enumerate(asm_text.split("\n")):
        m = re.match(r"^(_Z\w+):", l)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if l.startswith(".Lfunc_end"):
            out.append((name, body))
            name = None
            continue
        t = l.strip()
        m = re.match(r"^(\.LBB\d+_\d+):", t)
        if m:
            body.append((i + 1, m.group(1) + ":"))
        elif t and not t.startswith(";") and not t.startswith("."):
            body.append((i + 1, t))
    return out


def _vmcnt_of(t):
    m = re.search(r"vmcnt\((\d+)\)", t)
    if m:
        return int(m.group(1))
    return 0 if re.match(r"^s_waitcnt\s+0\s*$", t) else None


def _dst_sregs(t):
    """Scalar registers written by an instruction (its first operand), as a set."""
    parts = t.split(None, 1)
    if len(parts) < 2:
        return set()
    dst = parts[1].split(",")[0].strip()
    return _sregs(dst)


def _exec_step(t, st):
    """Abstract effect of one instruction on the scalar control state
    (exec known all-ones; SGPR pairs holding a mask saved while it was;
    64-bit SGPR pairs known to hold 0 or -1; vcc known zero / non-zero)."""
    full, saved, consts, vcc = st
    parts = t.split(None, 1)
    mn = parts[0]
    ops = [o.strip() for o in parts[1].split(";")[0].split(",")] if len(parts) > 1 else []
    dst = ops[0] if ops else ""
    written = _dst_sregs(t) if dst not in ("exec", "vcc") else set()
    if written:
        saved = frozenset(x for x in saved if not (_sregs(x) & written))
        consts = {k: v for k, v in consts.items() if not (_sregs(k) & written)}
    if dst == "exec":
        if mn == "s_mov_b64" and len(ops) > 1 and ops[1] == "-1":
            full = True
        elif mn == "s_or_b64" and len(ops) == 3 and "exec" in ops[1:]:
            other = ops[2] if ops[1] == "exec" else ops[1]
            full = True if other in saved else full
        else:
            full = False
        return full, saved, consts, vcc
    if mn == "s_mov_b64" and len(ops) == 2 and ops[1] == "exec":
        # a copy of exec, restored later with s_or_b64 exec, exec, <copy>
        return full, (saved | {dst}) if full else saved, consts, vcc
    if mn.startswith("s_") and "saveexec" in mn and ops:
        # saves the current exec into ops[0], then changes exec
        return False, (saved | {dst}) if full else saved, consts, vcc
    if mn == "s_mov_b64" and len(ops) == 2 and ops[1] in ("0", "-1") and dst.startswith("s["):
        consts = dict(consts)
        consts[dst] = int(ops[1])
    if dst == "vcc":
        vcc = None
        if mn in ("s_and_b64", "s_andn2_b64") and len(ops) == 3 and ops[1] == "exec" and ops[2] in consts:
            c = consts[ops[2]]
            if mn == "s_andn2_b64":
                c = ~c
            if c == 0:
                vcc = "zero"
            elif c == -1 and full:
                vcc = "nonzero"
    elif mn.startswith("v_") and ("vcc" in ops or mn.endswith("_e32") and ("cmp" in mn or "_co_" in mn
                                                                            or "addc" in mn or "subb" in mn)):
        vcc = None
    return full, saved, consts, vcc


def _edges(last, bi, nblocks, label_of, st):
    """Feasible successors of a block ending in `last` under control state st."""
    full, _, _, vcc = st
    if last.startswith("s_branch"):
        return [label_of[last.split()[-1]]]
    if last.startswith("s_endpgm"):
        return []
    fall = [bi + 1] if bi + 1 < nblocks else []
    if not last.startswith("s_cbranch"):
        return fall
    mn, tgt = last.split()[0], [label_of[last.split()[-1]]]
    if mn == "s_cbranch_execz" and full:
        return fall
    if mn == "s_cbranch_execnz" and full:
        return tgt
    if mn == "s_cbranch_vccnz" and vcc is not None:
        return tgt if vcc == "nonzero" else fall
    if mn == "s_cbranch_vccz" and vcc is not None:
        return tgt if vcc == "zero" else fall
    return tgt + fall


def vmcnt_stage_violations(asm_text):
    """Tagged waits that may release a stage before its loads have landed.

    The kernels' pipelined loads carry the stage they fill ("; ssd-stage k")
    and their explicit waits the stage they release ("; ssd-wait k" on an
    `s_waitcnt vmcnt(n)`). Loads and stores share the vmcnt counter and retire
    in issue order, so `vmcnt(n)` releases stage k only if at least n vector
    memory instructions were issued after stage k's last load. A forward
    dataflow over the control-flow graph keeps, per stage, the minimum of that
    count over all paths (every wait, the compiler's too, retires what it
    covers).

    Paths that need an all-zero exec mask where exec is known to be all ones
    (the fall-through of `s_cbranch_execnz`, the target of `s_cbranch_execz`)
    are not taken: the control-flow structurizer emits such edges for loop
    exits, and no wave runs them. Exec is known full at entry (whole waves)
    and after restoring a mask that was saved while it was full.

    Returns (violations, per-function (tagged loads, tagged waits)); a
    violation is (function, line, stage, n, count)."""
    bad, counts = [], {}
    for fname, body in _functions(asm_text):
        blocks, cur, label_of = [], [], {}
        for ln, t in body:
            if t.endswith(":"):
                if cur:
                    blocks.append(cur)
                cur = []
                label_of[t[:-1]] = len(blocks)
                continue
            cur.append((ln, t))
            if t.startswith("s_branch") or t.startswith("s_cbranch") or t.startswith("s_endpgm"):
                blocks.append(cur)
                cur = []
        if cur:
            blocks.append(cur)
        n_loads = sum(1 for blk in blocks for _, t in blk if "ssd-stage" in t)
        n_waits = sum(len(re.findall("ssd-wait", t)) for blk in blocks for _, t in blk)
        counts[fname] = (n_loads, n_waits)
        if not blocks:
            continue
        stages = sorted({int(m) for blk in blocks for _, t in blk for m in re.findall(r"ssd-stage (\d+)", t)})

        def key(st):
            f, sv, c, v = st
            return (f, sv, tuple(sorted(c.items())), v)

        # per block: control state -> per-stage minimum counts (paths are kept
        # apart by control state, merged only when it is the same)
        state_in = [dict() for _ in blocks]
        st0 = (True, frozenset(), {}, None)
        state_in[0][key(st0)] = (st0, {k: _INF for k in stages})
        work, found = [(0, key(st0))], {}
        while work:
            bi, ck = work.pop()
            st, d0 = state_in[bi][ck]
            d = dict(d0)
            for ln, t in blocks[bi]:
                if t.startswith("s_waitcnt"):
                    n = _vmcnt_of(t)
                    for ks_, ex_ in re.findall(r"ssd-wait (\d+)(?: excl (\d+))?", t) if n is not None else []:
                        k, excl = int(ks_), int(ex_ or 0)
                        if d.get(k, _INF) < n - excl:
                            old = found.get((ln, k))
                            if old is None or d[k] < old[4]:
                                found[(ln, k)] = (fname, ln, k, n - excl, d[k])
                    if n is not None:
                        for k in d:
                            if d[k] >= n:
                                d[k] = _INF
                    continue
                if _VMEM.match(t.split()[0]):
                    m = re.search(r"ssd-stage (\d+)", t)
                    if "ssd-export" not in t:
                        for k in d:
                            d[k] = min(_INF, d[k] + 1)
                    if m:
                        d[int(m.group(1))] = 0
                st = _exec_step(t, st)
            nk = key(st)
            for sb in _edges(blocks[bi][-1][1], bi, len(blocks), label_of, st):
                prev = state_in[sb].get(nk)
                if prev is None:
                    state_in[sb][nk] = (st, dict(d))
                    work.append((sb, nk))
                else:
                    merged = {k: min(prev[1][k], d[k]) for k in d}
                    if merged != prev[1]:
                        state_in[sb][nk] = (st, merged)
                        work.append((sb, nk))
        bad.extend(found.values())
    return bad, counts


def store_data_hazards(asm_text, need=2):
    """Stores of more than 8 bytes (dwordx3 / dwordx4) whose data registers a
    VALU instruction overwrites fewer than `need` wait states later (gfx940-
    family parts, gfx950 included, need two: the store may still be reading
    them; each instruction in between is one wait state, s_nop N is N + 1).
    Straight-line view; returns (line, store, writer) per hazard and the
    number of such stores seen."""
    ins = []
    for i, l in enumerate(asm_text.split("\n")):
        t = l.split(";")[0].strip() if not l.strip().startswith(";") else ""
        if t and not t.startswith(".") and not t.endswith(":"):
            ins.append((i + 1, t))
    bad, count = [], 0
    for k, (ln, t) in enumerate(ins):
        mn = t.split()[0]
        if not re.match(r"^(buffer|global|flat|scratch)_store_dwordx[34]$", mn):
            continue
        count += 1
        ops = t.split(None, 1)[1].split(",")
        m = re.search(r"v\[(\d+):(\d+)\]", ops[0] if mn.startswith("buffer") else ops[1])
        if not m:
            continue
        data = set(range(int(m.group(1)), int(m.group(2)) + 1))
        ws = 0
        for j in range(k + 1, len(ins)):
            if ws >= need:
                break
            nt = ins[j][1]
            if nt.startswith("v_") and " " in nt:
                dst = nt.split(None, 1)[1].split(",")[0]
                if _vregs(dst) & data:
                    bad.append((ln, t, nt))
                    break
            ws += int(nt.split()[1]) + 1 if nt.startswith("s_nop") else 1
    return bad, count


def kernel_resources(asm_text):
    """{kernel symbol: {field: value}} from the code object metadata of an assembly
    text (private_segment_fixed_size = scratch bytes per lane, vgpr_count, ...)."""
    out, cur = {}, None
    meta = asm_text[asm_text.find("amdhsa.kernels:"):]
    for line in meta.splitlines():
        s = line.strip()
        if s.startswith("- .") or s.startswith("-   ."):
            cur = {}
            s = s[1:].strip()
        if cur is None or ":" not in s or not s.startswith("."):
            continue
        k, v = s[1:].split(":", 1)
        v = v.strip()
        cur[k] = int(v) if v.lstrip("-").isdigit() else v
        if k == "name":
            out[v] = cur
    return out
