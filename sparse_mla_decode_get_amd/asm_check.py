"""Build-time check of the wait states around MFMA instructions in generated gfx950 assembly.

Part of the kernels' MFMAs are written as inline assembly, which the compiler's hazard recognizer
does not see into. This check reads the device assembly of such a kernel and reports every place
where fewer wait states separate two dependent instructions than gfx950 requires (values the
compiler itself inserts for these cases):
  * a VALU instruction writes a VGPR that an MFMA reads as an operand: 2 wait states;
  * an MFMA writes registers that a non-MFMA instruction then reads: 12 wait states for the
    8-pass v_mfma_f32_32x32x16_bf16 (a following MFMA reading them as its accumulator input is
    forwarded and needs none).
It also rejects, conservatively, an MFMA whose result registers overlap its A or B operand (inline
assembly outputs without an early-clobber constraint can be given such registers; the compiler's
own MFMAs never are). m0_outside_inline_asm() lists compiler-generated instructions that use m0.
Each instruction counts as one wait state, s_nop N as N + 1. Branches end the window conservatively
(the scan is linear over the text).
"""
import re

MFMA_WRITE_READ = 12
VALU_WRITE_MFMA = 2


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _instructions(text, kernel):
    lines = text.split("\n")
    start = next(i for i, l in enumerate(lines) if l.split(";")[0].strip() == kernel + ":")
    out = []
    for l in lines[start + 1:]:
        t = l.strip().split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        if t.endswith(":"):
            out.append(("label", t))
            continue
        out.append(("ins", t))
        if t.startswith("s_endpgm"):
            break
    return out


def _operands(t):
    parts = t.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o for o in re.split(r",\s*", parts[1]) if o]


def check(text, kernel):
    """Return a list of human-readable violations for `kernel` in assembly `text`."""
    ins = _instructions(text, kernel)
    problems = []
    for k, (kind, t) in enumerate(ins):
        if kind != "ins":
            continue
        op, ops = _operands(t)
        if op.startswith("v_mfma"):
            if _regs(ops[0]) & (_regs(ops[1]) | _regs(ops[2])):
                problems.append(f"MFMA result overlaps its A/B operand: {t}")
            reads = set()
            for o in ops[1:4]:
                reads |= _regs(o)
            ws = 0
            for j in range(k - 1, -1, -1):
                kj, u = ins[j]
                if kj == "label" or ws >= VALU_WRITE_MFMA:
                    break
                uop, uops = _operands(u)
                if uop.startswith("v_") and not uop.startswith("v_mfma") and uops and _regs(uops[0]) & reads:
                    problems.append(f"VALU write {ws} wait states before an MFMA read: {u} -> {t}")
                ws += int(uops[0]) + 1 if uop == "s_nop" else 1
            written = _regs(ops[0])
            ws = 0
            for j in range(k + 1, len(ins)):
                kj, u = ins[j]
                if kj == "label" or ws >= MFMA_WRITE_READ:
                    break
                uop, uops = _operands(u)
                if uop.startswith("v_mfma"):
                    # srcC forwarding is allowed; srcA/srcB reads of the result are not
                    if (_regs(uops[1]) | _regs(uops[2])) & written:
                        problems.append(f"MFMA result read as A/B {ws} wait states later: {t} -> {u}")
                elif uop.startswith(("v_", "ds_", "global_", "buffer_")) and any(_regs(o) & written for o in uops):
                    problems.append(f"MFMA result used {ws} wait states later: {t} -> {u}")
                ws += int(uops[0]) + 1 if uop == "s_nop" else 1
    return problems


def m0_outside_inline_asm(text, kernel):
    """Instructions of `kernel` outside inline-assembly blocks that name m0. The kernels' LDS copies
    set m0 inside their own assembly and leave it set, which is only sound while no
    compiler-generated instruction relies on m0."""
    lines = text.split("\n")
    start = next(i for i, l in enumerate(lines) if l.split(";")[0].strip() == kernel + ":")
    out, in_asm = [], False
    for l in lines[start + 1:]:
        if ";;#ASMSTART" in l:
            in_asm = True
            continue
        if ";;#ASMEND" in l:
            in_asm = False
            continue
        t = l.split(";")[0].strip()
        if not in_asm and re.search(r"\bm0\b", t):
            out.append(f"m0 used outside inline assembly: {t}")
        if t.startswith("s_endpgm"):
            break
    return out


def kernels(text, name_part):
    """Mangled names of the kernels defined in `text` whose name contains `name_part`."""
    out = []
    for l in text.split("\n"):
        head = l.split(";")[0].strip()
        if head.endswith(":") and head.startswith("_Z") and name_part in head:
            out.append(head[:-1])
    return out
