"""Build-time check of the decode kernel's generated code.

The QK products of a tile (bf16, or fp8 with fp8 queries) are inline-assembly MFMAs chained through one VGPR
accumulator, and only the last link of a chain waits (inside its own
statement, with s_nop) until its result can be read. The compiler does not
know when an assembly MFMA's result arrives, so the kernel is only correct if
no instruction between two links -- nor between the last link and its wait --
reads or writes the accumulator registers. check_qk_chains() verifies that on
the gfx950 assembly of decode.hip; build() fails if it does not hold.
"""
import re

_MFMAS = ("v_mfma_f32_32x32x16_bf16", "v_mfma_f32_32x32x64_f8f6f4")
_REG = re.compile(r"([vas])\[(\d+):(\d+)\]|([vas])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return {r for r in out if r[0] in "va"}


def check_qk_chains(asm: str):
    """Return (chains, violations): the number of VGPR-accumulator MFMA chains
    found and a list of offending instruction lines. Several chains may be
    interleaved (one per query row block); each link's srcC must be exactly
    its chain's accumulator, and no other instruction may touch an open
    chain's registers before its last link (the one followed by s_nop 7)."""
    lines = [l.split(";", 1)[0].strip() for l in asm.splitlines()]
    chains, bad, active = 0, [], []   # active: register sets of open chains
    for i, l in enumerate(lines):
        if not l or l.startswith(".") or l.endswith(":"):
            continue
        mnem, _, ops = l.partition(" ")
        if mnem in _MFMAS and ops.strip().startswith("v["):
            dst = _regs(ops.split(",")[0])
            src_c = ops.split(",")[-1].strip()
            srcs = _regs(",".join(ops.split(",")[1:-1]))
            nxt = next((x for x in lines[i + 1:] if x and not x.startswith(".")), "")
            ends = nxt.startswith("s_nop 7")
            if src_c == "0":
                chains += 1
                if any(srcs & a or dst & a for a in active):
                    bad.append(f"{i}: {l} (a new chain touches an open chain)")
                if not ends:
                    active.append(dst)
                continue
            acc = _regs(src_c)
            if acc not in active:
                if any(acc & a for a in active) or any(dst & a for a in active):
                    bad.append(f"{i}: {l} (accumulator changed inside a chain)")
                continue
            active.remove(acc)
            if any(srcs & a or dst & a for a in active):
                bad.append(f"{i}: {l} (touches another open chain)")
            if not ends:
                active.append(dst)
            continue
        if not active or mnem.startswith("s_"):
            continue
        regs = _regs(ops)
        if any(regs & a for a in active):
            bad.append(f"{i}: {l}")
    return chains, bad


_WAIT_STATES = 2   # VALU write of a VGPR -> MFMA read of it as an operand


def check_valu_to_mfma(asm: str):
    """Return the assembly MFMA links (VGPR accumulators) that read an
    operand a VALU instruction wrote fewer than _WAIT_STATES wait states
    earlier: the compiler inserts no hazard wait states for inline assembly."""
    lines = [l.split(";", 1)[0].strip() for l in asm.splitlines()]
    bad = []
    for i, l in enumerate(lines):
        mnem, _, ops = l.partition(" ")
        if mnem not in _MFMAS or not ops.strip().startswith("v["):
            continue
        srcs = _regs(",".join(ops.split(",")[1:]))
        waits, k = 0, i - 1
        while k >= 0 and waits < _WAIT_STATES:
            t = lines[k]
            k -= 1
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            tm, _, tops = t.partition(" ")
            if tm == "s_nop":
                waits += int(tops.strip().split()[0], 0) + 1
                continue
            if tm.startswith("v_") and not tm.startswith("v_mfma") and _regs(tops.split(",")[0]) & srcs:
                bad.append(f"{i}: {l} (VALU write {k + 1}: {t})")
                break
            waits += 1
    return bad


_M0 = re.compile(r"\bm0\b")


def check_m0(asm: str):
    """Return the instructions that touch M0 other than the direct-to-LDS load
    sequences (s_mov_b32 m0, <sgpr>; s_nop 0; global_load_lds_*). Those
    sequences are inline assembly that sets M0 without declaring it, which is
    only safe while the compiler itself never keeps a value in M0."""
    lines = [l.split(";", 1)[0].strip() for l in asm.splitlines()]
    bad = []
    for i, l in enumerate(lines):
        if not l or l.startswith(".") or l.endswith(":") or not _M0.search(l):
            continue
        mnem, _, ops = l.partition(" ")
        if mnem == "s_mov_b32" and ops.strip().startswith("m0,"):
            nxt = [x for x in lines[i + 1:i + 4] if x and not x.startswith(".")]
            if len(nxt) >= 2 and nxt[0].startswith("s_nop 0") and nxt[1].startswith("global_load_lds_"):
                continue
        bad.append(f"{i}: {l}")
    return bad


def _kernel_bodies(asm: str):
    """(name, lines) of each kernel function in the assembly."""
    lines = asm.splitlines()
    out, cur, start = [], None, 0
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):\s*(;.*)?$", l)
        if m:
            cur, start = m.group(1), i
        elif cur and l.strip().startswith("s_endpgm"):
            out.append((cur, lines[start:i + 1]))
            cur = None
    return out


def check_scratch_in_step_loops(asm: str):
    """Return the scratch (spill) accesses that sit inside an innermost loop
    whose body holds MFMA instructions: the per-tile step loops of the
    decode kernel. A spill reload there is a vector-memory access whose wait
    would also wait for the tile loads in flight. Loops come from the
    compiler's own loop comments on each basic block ("=>This Inner Loop
    Header", "in Loop: Header=..."), so code after a loop that the layout
    reaches by a backward branch is not taken for a loop body. A kernel with
    backward branches but no loop comments is reported as such."""
    bad = []
    for name, body in _kernel_bodies(asm):
        code = [l.split(";", 1)[0].strip() for l in body]
        loop_of, inner, cur, annotated = [], set(), None, False
        for i, l in enumerate(body):
            m = re.match(r"^(\.LBB\w+|; %bb\.\d+):(.*)$", l)
            if m:
                label, comment = m.group(1), m.group(2)
                after = body[i + 1] if i + 1 < len(body) else ""
                after = after if re.match(r"^\s*;", after) else ""
                note = comment + " " + after
                header = label[2:] if label.startswith(".L") else None
                if re.search(r"=>\s*This Inner Loop Header", note):
                    cur, annotated = header, True
                    inner.add(header)
                elif re.search(r"=>\s*This Loop Header", note):
                    cur, annotated = header, True
                else:
                    h = re.search(r"in Loop: Header=(BB\w+)", note)
                    cur = h.group(1) if h else None
            loop_of.append(cur)
        labels = {c[:-1] for c in code if re.match(r"^\.LBB\w+:$", c)}
        backward = any(re.match(r"^s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", c) for c in code) and labels
        if backward and not annotated and any(c.startswith("v_mfma") for c in code):
            bad.append(f"{name}: no loop comments in the assembly; cannot place the spills")
            continue
        mfma_loops = {loop_of[i] for i, c in enumerate(code) if c.startswith("v_mfma") and loop_of[i] in inner}
        for i, c in enumerate(code):
            if c.startswith("scratch_") and loop_of[i] in mfma_loops:
                bad.append(f"{name}: {i}: {c}")
    return bad


_DECODE_FLAGS = re.compile(r"decode_kernelILb([01])ELb([01])ELb([01])ELb([01])E")


def check_waits_behind_tile_loads(asm: str):
    """Return the vector-memory waits the compiler inserted (s_waitcnt vmcnt
    outside inline assembly) while direct-to-LDS loads may be in flight: after
    a global_load_lds with no hand-written vmcnt(0) in between, in program
    order. The kernel counts its tile and query loads with waits of its own;
    a wait the compiler adds is for a spill reload or another vector load,
    and since the vector-memory counter is in order it also waits for every
    tile load issued before that load. Program order stands in for the
    control-flow graph. Checked in every decode kernel without fp8 PV
    products: with split bf16 queries the fp8-PV kernel's item head reloads
    16 spilled query registers behind its first tile loads."""
    bad = []
    for name, body in _kernel_bodies(asm):
        m = _DECODE_FLAGS.search(name)
        if not m or m.group(4) == "1":
            continue
        in_asm, pending = False, False
        for i, l in enumerate(body):
            if ";;#ASMSTART" in l:
                in_asm = True
                continue
            if ";;#ASMEND" in l:
                in_asm = False
                continue
            c = l.split(";", 1)[0].strip()
            if not c:
                continue
            if c.startswith("global_load_lds"):
                pending = True
            elif c.startswith("s_waitcnt") and "vmcnt" in c:
                if in_asm:
                    if re.search(r"vmcnt\(0\)", c):
                        pending = False
                elif pending:
                    bad.append(f"{name}: {i}: {c}")
    return bad
