"""Build-time check of the decode kernel's generated code.

The QK products of a tile are inline-assembly MFMAs chained through one VGPR
accumulator, and only the last link of a chain waits (inside its own
statement, with s_nop) until its result can be read. The compiler does not
know when an assembly MFMA's result arrives, so the kernel is only correct if
no instruction between two links -- nor between the last link and its wait --
reads or writes the accumulator registers. check_qk_chains() verifies that on
the gfx950 assembly of decode.hip; build() fails if it does not hold.
"""
import re

_MFMA = "v_mfma_f32_32x32x16_bf16"
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
    found and a list of offending instruction lines."""
    lines = [l.split(";", 1)[0].strip() for l in asm.splitlines()]
    chains, bad, active = 0, [], None
    for i, l in enumerate(lines):
        if not l or l.startswith(".") or l.endswith(":"):
            continue
        mnem, _, ops = l.partition(" ")
        if mnem == _MFMA and ops.strip().startswith("v["):
            dst = _regs(ops.split(",")[0])
            src_c = ops.split(",")[-1].strip()
            if active is None or src_c == "0":
                chains += 1
            elif _regs(src_c) != active:
                bad.append(f"{i}: {l} (accumulator changed inside a chain)")
            nxt = next((x for x in lines[i + 1:] if x and not x.startswith(".")), "")
            active = None if nxt.startswith("s_nop 7") else dst
            continue
        if active is None or mnem.startswith("s_"):
            continue
        if _regs(ops) & active:
            bad.append(f"{i}: {l}")
    return chains, bad
