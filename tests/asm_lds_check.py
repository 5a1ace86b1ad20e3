"""Static check of LDS reads issued in inline assembly (the prefill tile's V
operands): the compiler does not track them, so nothing may touch their
destination registers before an `s_waitcnt` that waits for every LDS
operation (lgkmcnt(0)).  Scans the AMD assembly of a build, kernel by kernel,
in text order; a use reached only through a loop's back edge is not seen
(the kernel waits for its reads within the step that issues them)."""
import re

_ASM_READ = re.compile(r"^\s*(ds_read2st64_b64|ds_read_b128)\s+(v\[(\d+):(\d+)\]|v(\d+))")
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_WAIT0 = re.compile(r"^\s*s_waitcnt\b.*lgkmcnt\(0\)")
_FUNC = re.compile(r"^(_Z\w+):")


def _regs(text):
    out = set()
    for a, b, c in _REG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def violations(asm_text):
    """(kernel, line number, instruction) of every instruction that reads or
    writes a register an inline-assembly LDS read is still filling."""
    bad = []
    kernel = None
    pending = set()
    in_asm = False
    for n, line in enumerate(asm_text.splitlines(), 1):
        m = _FUNC.match(line)
        if m:
            kernel, pending = m.group(1), set()
            continue
        s = line.split(";")[0].rstrip()
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        if not s.strip() or s.strip().startswith(".") or s.strip().endswith(":"):
            continue
        if _WAIT0.match(s):
            pending = set()
            continue
        r = _ASM_READ.match(s)
        if in_asm and r:
            a, b, c = r.group(3), r.group(4), r.group(5)
            dst = set(range(int(a), int(b) + 1)) if a is not None else {int(c)}
            # its address operand may be read; its destination is now pending
            src = _regs(s[r.end(2):])
            if src & pending:
                bad.append((kernel, n, s.strip()))
            pending |= dst
            continue
        if in_asm and s.strip().startswith("s_nop"):
            continue  # the operand hand-over after the wait (no register access)
        if _regs(s) & pending:
            bad.append((kernel, n, s.strip()))
    return bad


def asm_lds_reads(asm_text):
    """Number of inline-assembly LDS reads in the text."""
    return sum(1 for line in asm_text.splitlines() if _ASM_READ.match(line.split(";")[0]))
