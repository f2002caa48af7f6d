"""Static check of compiled gfx950 kernels: a vector memory instruction may
read a scalar register that a vector-ALU instruction wrote only after 5 wait
states in between.

The hardware does not interlock this case (the ISA's table of manually
inserted wait states lists "VALU writes SGPR, then VMEM reads that SGPR" at
5). The compiler inserts the wait states in its own code but not in front of
inline assembly, which it does not look into: a scalar base address made
with v_readfirstlane and passed to an assembly store as its saddr operand is
then read too early, and the store writes to a stale address.

Model: each function of the assembly is scanned in program order; an
instruction counts one wait state, `s_nop N` counts N + 1. A vector-ALU
instruction writes the scalar registers of its scalar destination (the first
operand of v_readfirstlane, v_readlane and the compares; the carry-out
operand of the add / subtract / multiply-add forms that have one). A vector
memory instruction (global_, buffer_, flat_, scratch_) reads every scalar
register among its operands (saddr, resource, soffset). A read with fewer
than 5 wait states since the last such write of one of its registers is
reported. Labels are passed through as fall-through, so a write on the path
into a block counts; a write reached only by a jump is not followed (the
hazard this check is for sits in straight-line code)."""
from __future__ import annotations

import re

_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_FUNC = re.compile(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$")
_NEEDED = 5
# vector-ALU opcodes whose second operand is a scalar destination (carry out)
_CARRY_DST = ("v_add_co_u32", "v_sub_co_u32", "v_subrev_co_u32", "v_addc_co_u32",
              "v_subb_co_u32", "v_subbrev_co_u32", "v_mad_u64_u32", "v_mad_i64_i32",
              "v_div_scale_f32", "v_div_scale_f64")
_VMEM = ("global_", "buffer_", "flat_", "scratch_")


def _sregs(text: str) -> set[int]:
    out: set[int] = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _operands(rest: str) -> list[str]:
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return ops


def _instructions(lines):
    """(opcode, operand text, line) for the instruction lines, in order."""
    for raw in lines:
        line = raw.split(";", 1)[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        parts = line.split(None, 1)
        yield parts[0], parts[1] if len(parts) > 1 else "", line


def check_function(lines) -> list[str]:
    written: dict[int, tuple[int, str]] = {}  # sreg -> (wait-state clock at the write, line)
    clock = 0
    found = []
    for op, rest, line in _instructions(lines):
        ops = _operands(rest)
        if op.startswith(_VMEM):
            for r in sorted(_sregs(" ".join(ops))):
                if r in written and clock - written[r][0] - 1 < _NEEDED:
                    found.append(f"{written[r][1]}  ->  {line}")
                    break
        if op.startswith("v_"):
            dst: set[int] = set()
            if ops and _sregs(ops[0]) and not ops[0].startswith("v"):
                if op.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
                    dst |= _sregs(ops[0])
            if op.startswith(_CARRY_DST) and len(ops) > 1:
                dst |= _sregs(ops[1])
            for r in dst:
                written[r] = (clock, line)
        if op == "s_nop":
            clock += int(rest.strip(), 0) + 1
        else:
            clock += 1
    return found


def check_assembly(text: str) -> dict[str, list[str]]:
    """Function name -> the hazardous (write -> read) pairs, for every
    function of a gfx950 assembly listing."""
    out: dict[str, list[str]] = {}
    name, body = None, []
    for raw in text.splitlines():
        m = _FUNC.match(raw.strip())
        if m and not raw.startswith((" ", "\t")) and not m.group(1).startswith(".L"):
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if raw.strip().startswith(".Lfunc_end"):
            h = check_function(body)
            if h:
                out[name] = h
            name = None
            continue
        body.append(raw)
    return out
