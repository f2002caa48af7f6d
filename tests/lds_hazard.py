"""Static check of compiled gfx950 kernels: no instruction may read or write a
VGPR while an LDS read into that VGPR is still in flight.

The main loop issues its LDS operand reads as inline assembly and waits for
them with explicit lgkmcnt values, so the compiler treats each read's result
as written when the read is issued. If register allocation then copies such a
value (or writes the register) before the matching wait, the copy holds stale
data and results are silently wrong. This checker walks the control-flow
graph of every kernel in the assembly and reports such accesses.

Model: LDS reads return in order; `s_waitcnt lgkmcnt(N)` leaves at most the N
most recent LDS operations outstanding. State per point = the list of
destination register sets of the outstanding LDS reads, oldest first. It is a
"must" analysis: at a join only what is in flight on every incoming path is
kept (lists aligned at the most recent entry, sets intersected), so a report
is a read that is in flight whichever way the code got there; an access that
is hazardous on one path only can go unreported. An LDS read whose
destination overlaps an older outstanding read is allowed (returns are in
order)."""
from __future__ import annotations

import re

_LABEL = re.compile(r"^(\.LBB\w+|\.Ltmp\w*):")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def _regs(text: str) -> set[int]:
    out: set[int] = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split_ops(rest: str) -> list[str]:
    # operands up to the first modifier-only token (offset:, glc, lds, ...)
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


def _classify(line: str):
    """-> (kind, dst_regs, src_regs, lgkm_wait or None)."""
    parts = line.split(None, 1)
    op = parts[0]
    rest = parts[1] if len(parts) > 1 else ""
    rest = rest.split(";")[0]
    if op == "s_waitcnt":
        m = _LGKM.search(rest)
        return "wait", set(), set(), int(m.group(1)) if m else None
    if op.startswith("ds_read") or op.startswith("ds_load"):
        ops = _split_ops(rest)
        return "lds_read", _regs(ops[0]) if ops else set(), _regs(" ".join(ops[1:])), None
    if op.startswith(("ds_write", "ds_store", "ds_add", "ds_swizzle", "ds_bpermute",
                      "ds_permute")):
        ops = _split_ops(rest)
        if op.startswith(("ds_swizzle", "ds_bpermute", "ds_permute")):
            return "lds_other", _regs(ops[0]) if ops else set(), _regs(" ".join(ops[1:])), None
        return "lds_other", set(), _regs(rest), None
    if op.startswith(("buffer_store", "global_store", "scratch_store", "flat_store")):
        return "other", set(), _regs(rest), None
    if op.startswith(("buffer_load", "global_load", "scratch_load", "flat_load",
                      "buffer_atomic", "global_atomic")):
        ops = _split_ops(rest)
        if " lds" in " " + rest or rest.rstrip().endswith("lds"):
            return "other", set(), _regs(rest), None
        return "other", _regs(ops[0]) if ops else set(), _regs(" ".join(ops[1:])), None
    if op.startswith("v_"):
        ops = _split_ops(rest)
        if not ops:
            return "other", set(), set(), None
        if op.startswith(("v_cmp", "v_readfirstlane", "v_readlane")) and not op.startswith(
                "v_cmpx"):
            return "other", set(), _regs(" ".join(ops)), None
        return "other", _regs(ops[0]), _regs(" ".join(ops[1:])), None
    return "other", set(), set(), None


def _meet(a: list[frozenset], b: list[frozenset]) -> list[frozenset]:
    n = min(len(a), len(b))
    a, b = a[len(a) - n:], b[len(b) - n:]
    return [x & y for x, y in zip(a, b)]


def check_function(lines: list[str]) -> list[str]:
    """Hazards in one function's instruction lines (labels included)."""
    # Basic blocks: a label starts one, and every branch ends one (the
    # fall-through block after a conditional branch has no label of its own).
    blocks: list[tuple[str, list[str]]] = [("<entry>", [])]
    for raw in lines:
        t = raw.strip()
        if not t or t.startswith(";") or t.startswith("."):
            m = _LABEL.match(t)
            if m:
                blocks.append((m.group(1), []))
            continue
        blocks[-1][1].append(t)
        if t.startswith(("s_branch", "s_cbranch")):
            blocks.append((f"<after {t}>", []))
    index = {name: i for i, (name, _) in enumerate(blocks)}

    def succs(i: int) -> list[int]:
        body = blocks[i][1]
        out = []
        last = body[-1] if body else ""
        m = re.match(r"s_(c?branch)\w*\s+(\.LBB\w+)", last)
        if m and m.group(2) in index:
            out.append(index[m.group(2)])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            out.append(i + 1)
        return out

    state_in: dict[int, list[frozenset]] = {0: []}
    work = [0]
    hazards: list[str] = []
    seen_hazard: set[tuple[int, str]] = set()
    while work:
        i = work.pop()
        st = list(state_in[i])
        for t in blocks[i][1]:
            kind, dst, src, wait = _classify(t)
            if kind == "wait":
                if wait is not None:
                    st = st[len(st) - wait:] if wait < len(st) else st
                    if wait == 0:
                        st = []
                continue
            pending = frozenset().union(*st) if st else frozenset()
            touched = (src | (dst if kind != "lds_read" else set())) & pending
            if touched and (i, t) not in seen_hazard:
                seen_hazard.add((i, t))
                hazards.append(f"{blocks[i][0]}: '{t}' touches v{sorted(touched)} "
                               f"while an LDS read into it is in flight")
            if kind in ("lds_read", "lds_other"):
                st.append(frozenset(dst))
        for j in succs(i):
            new = st if j not in state_in else _meet(state_in[j], st)
            if j not in state_in or new != state_in[j]:
                state_in[j] = new
                work.append(j)
    return hazards


def check_assembly(text: str, name_filter: str = "") -> dict[str, list[str]]:
    """Hazards per function of a gfx950 assembly listing."""
    out: dict[str, list[str]] = {}
    parts = re.split(r"\n(?=_Z\S+:)", text)
    for part in parts:
        m = re.match(r"(_Z\S+):", part)
        if not m or name_filter not in m.group(1):
            continue
        end = part.find(".Lfunc_end")
        lines = part[: end if end > 0 else len(part)].split("\n")[1:]
        h = check_function(lines)
        if h:
            out[m.group(1)] = h
    return out
