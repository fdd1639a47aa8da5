"""Wait-state check of inline-asm matrix instructions in gfx950 device assembly.

hipcc pads the register dependencies of the MFMAs it schedules itself with
independent instructions or ``s_nop``, but an instruction written inside an
inline-asm block is opaque to it: a VALU write of an operand just before an
inline-asm MFMA, or an access of its result too soon after it, gets no
padding, and the MFMA then reads a stale operand or the reader a stale result.
Which pairs end up close depends on the compiler's schedule, so any change to
a kernel can create one.  ``check`` scans hipcc's device assembly (``-S``) for
such pairs; the library build refuses code with any.

Distances are in wait states: an instruction counts 1, ``s_nop n`` counts
n + 1, labels nothing; every path through conditional branches is followed.
The required distances are the ones hipcc itself inserts on gfx950 around
the MFMAs it emits (read off its own output for these instructions):

* a VALU write of a register, then an MFMA reading it (A, B or C): 2;
* an MFMA, then a non-MFMA instruction reading or writing its result
  registers, or a later MFMA reading them as A or B or as part of a
  differently placed C: 8 for ``v_mfma_f32_16x16x32_bf16`` (4 passes), 12
  for ``v_mfma_f32_32x32x16_bf16`` (8 passes), 20 for any other MFMA;
* an MFMA reading C, then a VALU write of those registers: the same as its
  result (more than hipcc asks for, so safe).

A pair is checked when at least one side sits inside an inline-asm block; the
compiler already covers pairs of its own instructions.  An MFMA reads its A and
B operands when it issues, so writing them right after it needs no padding
(hipcc leaves none either) and is not reported.
"""
from __future__ import annotations

import re
from dataclasses import dataclass

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_RESULT_WAIT = {"v_mfma_f32_16x16x32_bf16": 8, "v_mfma_f32_32x32x16_bf16": 12}
_DEFAULT_RESULT_WAIT = 20
_VALU_TO_MFMA = 2


@dataclass(frozen=True)
class Finding:
    kernel: str
    rule: str       # "valu->mfma", "mfma->read", "mfma->mfma" or "srcc->write"
    distance: int   # wait states between the two instructions
    needed: int
    first: str
    second: str

    def __str__(self):
        return (f"{self.kernel}: {self.rule} {self.distance} < {self.needed} wait states\n"
                f"    {self.first}\n    {self.second}")


@dataclass
class _Ins:
    text: str
    op: str
    ops: list
    in_asm: bool
    label: str | None = None  # set for label lines


def _regs(s: str) -> set:
    out = set()
    for m in _REG.finditer(s):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _split(text: str):
    op, _, rest = text.partition(" ")
    ops, depth, cur = [], 0, ""
    for ch in rest:
        depth += (ch == "[") - (ch == "]")
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return op, ops


def _written(ins: _Ins) -> set:
    """Vector / accumulation registers the instruction writes."""
    op, ops = ins.op, ins.ops
    if not ops or op.startswith("s_"):
        return set()
    if op.startswith("v_"):
        if op.startswith(("v_readlane", "v_readfirstlane")) or (op.startswith("v_cmp") and not op.startswith("v_cmpx")):
            return set()
        return _regs(ops[0])
    if op.startswith(("ds_read", "ds_load", "ds_bpermute", "ds_permute", "ds_swizzle")) or "_rtn" in op:
        return _regs(ops[0])
    if op.startswith(("buffer_load", "global_load", "flat_load", "scratch_load")):
        return set() if "lds" in ins.text.split() else _regs(ops[0])
    return set()


def _accessed(ins: _Ins) -> set:
    return set().union(*(_regs(o) for o in ins.ops)) if ins.ops and not ins.op.startswith("s_") else set()


def _cost(ins: _Ins) -> int:
    if ins.label is not None:
        return 0
    if ins.op == "s_nop":
        return int(ins.ops[0], 0) + 1 if ins.ops else 1
    return 1


def _functions(asm: str):
    """{kernel symbol: [instructions]} from hipcc's device assembly."""
    funcs, cur, in_asm = {}, None, False
    for raw in asm.splitlines():
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^([A-Za-z_$][\w$.]*):", s)
        if m and not s.startswith(".L"):
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.L\w+):", s)
        if m:
            funcs[cur].append(_Ins(s, "", [], False, label=m.group(1)))
            continue
        text = s.split(";", 1)[0].strip()
        if not text or text.startswith("."):
            continue
        op, ops = _split(text)
        funcs[cur].append(_Ins(text, op, ops, in_asm))
    return {k: v for k, v in funcs.items() if any(i.op.startswith("v_mfma") for i in v)}


def _cfg(body):
    where = {ins.label: i for i, ins in enumerate(body) if ins.label is not None}
    succ = []
    for i, ins in enumerate(body):
        if ins.op == "s_branch":
            succ.append([where[ins.ops[0]]] if ins.ops and ins.ops[0] in where else [])
        elif ins.op.startswith("s_cbranch"):
            nxt = [i + 1] if i + 1 < len(body) else []
            succ.append(nxt + ([where[ins.ops[0]]] if ins.ops and ins.ops[0] in where else []))
        elif ins.op in ("s_endpgm", "s_setpc_b64"):
            succ.append([])
        else:
            succ.append([i + 1] if i + 1 < len(body) else [])
    pred = [[] for _ in body]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return succ, pred


def _walk(start, edges, body, budget):
    """(index, wait states between start and it) for every instruction within
    budget along edges, nearest distance per index."""
    best, stack = {}, [(j, 0) for j in edges[start]]
    while stack:
        i, d = stack.pop()
        if d >= budget or best.get(i, budget) <= d:
            continue
        best[i] = d
        for j in edges[i]:
            stack.append((j, d + _cost(body[i])))
    return best


def check_kernel(name: str, body) -> list:
    succ, pred = _cfg(body)
    found = []
    for m, ins in enumerate(body):
        if not ins.op.startswith("v_mfma") or len(ins.ops) < 4:
            continue
        dst = _regs(ins.ops[0])
        a_b = _regs(ins.ops[1]) | _regs(ins.ops[2])
        c = _regs(ins.ops[3])
        need = _RESULT_WAIT.get(ins.op, _DEFAULT_RESULT_WAIT)
        # writes of its operands before it
        for i, d in _walk(m, pred, body, _VALU_TO_MFMA).items():
            other = body[i]
            if not (ins.in_asm or other.in_asm) or not other.op.startswith("v_") or other.op.startswith("v_mfma"):
                continue
            if _written(other) & (a_b | c):
                found.append(Finding(name, "valu->mfma", d, _VALU_TO_MFMA, other.text, ins.text))
        # uses of its result after it
        for i, d in _walk(m, succ, body, need).items():
            other = body[i]
            if not (ins.in_asm or other.in_asm) or other.label is not None:
                continue
            if other.op.startswith("v_mfma") and len(other.ops) >= 4:
                c2 = _regs(other.ops[3])
                if (_regs(other.ops[1]) | _regs(other.ops[2])) & dst or (c2 & dst and c2 != dst):
                    found.append(Finding(name, "mfma->mfma", d, need, ins.text, other.text))
                continue
            if _accessed(other) & dst:
                found.append(Finding(name, "mfma->read", d, need, ins.text, other.text))
            elif _written(other) & (c - dst):
                found.append(Finding(name, "srcc->write", d, need, ins.text, other.text))
    return found


def check(asm: str) -> list:
    """Every finding in one device assembly file's text."""
    out = []
    for name, body in _functions(asm).items():
        out.extend(check_kernel(name, body))
    return out
