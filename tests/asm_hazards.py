"""Static checks on the gfx950 assembly of the HIP kernels.

The GEMM kernels issue their MFMAs as inline asm with the accumulators tied in
AGPRs.  The compiler's hazard recognizer does not see the operands of inline
asm as MFMA operands, so the wait states that CDNA3/CDNA4 require around an
MFMA are not inserted for them; the kernels arrange them by construction
(explicit s_nop, barriers, enough independent MFMAs in between).  This module
parses the assembly the compiler produces and checks, along every control-flow
path, the rules the kernels rely on:

  * no scratch (spill) traffic at all in a kernel that contains MFMAs;
  * a VALU write of a VGPR/AGPR is at least VALU_TO_MFMA wait states before an
    MFMA that reads it (the CDNA3 ISA's "VALU write VGPR, MFMA read" rule);
  * an MFMA's result registers are neither read nor written by a non-MFMA
    instruction, nor read as a source operand other than its own accumulator
    by another MFMA, within MFMA_RESULT wait states of it (16-pass worst case
    plus margin); a later MFMA accumulating into exactly the same registers is
    the supported back-to-back form;
  * a VALU instruction writes an MFMA's accumulator-input registers no
    sooner than MFMA_RESULT wait states after it (write-after-read).

Only pairs in which at least one instruction comes from inline asm are
checked: between two compiler-generated instructions the compiler's own hazard
recognizer, which knows each MFMA's pass count, inserts the waits.

Wait states are counted as the hazard recognizer does: one per instruction,
N + 1 for ``s_nop N``.  The walk is conservative at branches: every
predecessor path is followed.
"""
from __future__ import annotations

import re
import subprocess
from dataclasses import dataclass, field

VALU_TO_MFMA = 2
MFMA_RESULT = 18

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_MODS = re.compile(r"\s+(op_sel|op_sel_hi|cbsz|blgp|abid|neg_lo|neg_hi|offset|offen|idxen|lds|glc|slc|nt|sc0|sc1)\b.*$")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            lo, hi = int(m.group(2)), int(m.group(3))
            out.update((kind, r) for r in range(lo, hi + 1))
    return out


@dataclass
class Instr:
    mnem: str
    text: str
    writes: set = field(default_factory=set)
    reads: set = field(default_factory=set)
    srcc: set = field(default_factory=set)   # MFMA accumulator input
    srcab: set = field(default_factory=set)  # MFMA other sources (A, B, scales)
    inline: bool = False                     # emitted from an inline asm statement

    @property
    def is_mfma(self) -> bool:
        return self.mnem.startswith("v_mfma")

    @property
    def is_valu(self) -> bool:
        return self.mnem.startswith("v_") and not self.is_mfma

    @property
    def wait_states(self) -> int:
        if self.mnem == "s_nop":
            return int(self.text.split()[1], 0) + 1
        return 1


def _parse_instr(line: str) -> Instr:
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    mnem = parts[0]
    ops = parts[1] if len(parts) > 1 else ""
    ins = Instr(mnem, body)
    core = _MODS.sub("", ops)
    pieces = [p.strip() for p in core.split(",")] if core else []
    if ins.is_mfma:
        ins.writes = _regs(pieces[0])
        ins.srcab = set().union(*[_regs(p) for p in pieces[1:3]]) | set().union(*[_regs(p) for p in pieces[4:]])
        ins.srcc = _regs(pieces[3]) if len(pieces) > 3 else set()
        ins.reads = ins.srcab | ins.srcc
        return ins
    no_dst = (mnem.startswith(("s_", "ds_write", "ds_store", "global_store", "buffer_store", "scratch_store",
                               "flat_store", "exp")) or (" lds" in " " + ops and "load" in mnem)
              or mnem.startswith(("v_cmp_", "v_cmpx_", "v_readfirstlane", "v_readlane")))
    if pieces and not no_dst:
        ins.writes = _regs(pieces[0])
        ins.reads = set().union(*[_regs(p) for p in pieces[1:]]) if len(pieces) > 1 else set()
    else:
        ins.reads = _regs(core)
    return ins


@dataclass
class Function:
    name: str
    instrs: list
    preds: list
    scratch_bytes: int


def parse_functions(asm: str) -> list:
    funcs = []
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S*|[A-Za-z_]\w*):\s*(;.*)?$", lines[i])
        if not m or lines[i].startswith("."):
            i += 1
            continue
        name = m.group(1)
        instrs, labels_at, branches = [], {}, []
        pending = []
        in_asm = False
        j = i + 1
        while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
            ln = lines[j]
            lm = re.match(r"^(\.LBB\w+):", ln)
            if ";;#ASMSTART" in ln:
                in_asm = True
            elif ";;#ASMEND" in ln:
                in_asm = False
            elif lm:
                pending.append(lm.group(1))
            else:
                s = ln.strip()
                if s and not s.startswith((";", ".")) and re.match(r"^[a-z_][a-z0-9_]*", s):
                    for lab in pending:
                        labels_at[lab] = len(instrs)
                    pending = []
                    ins = _parse_instr(s)
                    ins.inline = in_asm
                    if ins.mnem.startswith(("s_cbranch", "s_branch")):
                        branches.append((len(instrs), ins.text.split()[1]))
                    instrs.append(ins)
            j += 1
        if not instrs:
            i = j + 1
            continue
        preds = [[] for _ in instrs]
        for k in range(1, len(instrs)):
            if instrs[k - 1].mnem not in ("s_branch", "s_endpgm", "s_setpc_b64"):
                preds[k].append(k - 1)
        for src, lab in branches:
            if lab in labels_at:
                preds[labels_at[lab]].append(src)
        scratch = 0
        tail = "\n".join(lines[j:j + 400])
        sm = re.search(r"\.private_segment_fixed_size:\s*(\d+)", tail) or \
            re.search(r"ScratchSize:\s*(\d+)", tail)
        if sm:
            scratch = int(sm.group(1))
        funcs.append(Function(name, instrs, preds, scratch))
        i = j + 1
    return funcs


def _walk_back(f: Function, start: int, limit: int):
    """Yield (j, d): predecessors j of instruction `start` on any path, with d
    the wait states between j and `start` (d < limit)."""
    seen = {}
    stack = [(p, 0) for p in f.preds[start]]
    while stack:
        j, d = stack.pop()
        if d >= limit or seen.get(j, limit + 1) <= d:
            continue
        seen[j] = d
        yield j, d
        nd = d + f.instrs[j].wait_states
        for p in f.preds[j]:
            stack.append((p, nd))


def check_function(f: Function) -> list:
    problems = []
    has_mfma = any(ins.is_mfma for ins in f.instrs)
    if not has_mfma:
        return problems
    if f.scratch_bytes:
        problems.append("%s: scratch size %d bytes with MFMAs" % (f.name, f.scratch_bytes))
    for k, ins in enumerate(f.instrs):
        if ins.mnem.startswith("scratch_"):
            problems.append("%s: spill instruction %r" % (f.name, ins.text))
    for k, ins in enumerate(f.instrs):
        if not (ins.reads or ins.writes):
            continue
        for j, d in _walk_back(f, k, MFMA_RESULT):
            p = f.instrs[j]
            if not (p.inline or ins.inline):
                continue  # both compiler-generated: its hazard recognizer covers them
            if p.is_mfma:
                if ins.is_mfma:
                    if p.writes & ins.srcab and d < MFMA_RESULT:
                        problems.append("%s: MFMA result read as source %d wait states later: %r -> %r"
                                        % (f.name, d, p.text, ins.text))
                    ov = p.writes & ins.srcc
                    if ov and ins.srcc != p.writes and d < MFMA_RESULT:
                        problems.append("%s: partial accumulator overlap %d wait states later: %r -> %r"
                                        % (f.name, d, p.text, ins.text))
                else:
                    if (p.writes & (ins.reads | ins.writes)) and d < MFMA_RESULT:
                        problems.append("%s: MFMA result touched %d wait states later: %r -> %r"
                                        % (f.name, d, p.text, ins.text))
                    if ins.is_valu and (p.srcc & ins.writes) and d < MFMA_RESULT:
                        problems.append("%s: MFMA accumulator input overwritten %d wait states later: %r -> %r"
                                        % (f.name, d, p.text, ins.text))
            elif p.is_valu and ins.is_mfma:
                if p.writes & ins.reads and d < VALU_TO_MFMA:
                    problems.append("%s: VALU write read by MFMA %d wait states later: %r -> %r"
                                    % (f.name, d, p.text, ins.text))
    return problems


def compile_to_asm(src: str, flags: list, hipcc: str) -> str:
    cmd = [hipcc] + [f for f in flags if f != "-fPIC"] + ["--cuda-device-only", "-S", src, "-o", "-"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, res.stderr))
    return res.stdout
