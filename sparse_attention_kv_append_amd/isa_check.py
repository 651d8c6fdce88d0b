"""Static checks of the built gfx950 code: counted LDS waits and matrix results.

Several kernels issue LDS reads as inline assembly and wait for them with
counted `s_waitcnt lgkmcnt(N)` placed where the data is first needed, so
that reads run ahead of the matrix instructions that consume them. The
compiler does not know that the destination registers of such a read are
written asynchronously: it may copy, spill or reuse them before the wait,
and the copy then reads whatever the register held before the data arrived.

This module compiles a source to device assembly and proves, over every
path of each kernel's control flow graph, that no instruction touches a
register an LDS read still owes. LDS operations complete in issue order, so
after `lgkmcnt(N)` every LDS operation followed by at least N later LDS
operations has completed, whatever scalar-memory loads are mixed in (they
share the counter but can only make the count larger). The abstract state
maps each pending LDS read (by instruction) to the fewest later LDS
operations seen on any path, and paths merge by taking the minimum.

The same walk checks the distance from each matrix instruction to the first
non-matrix instruction that reads or overwrites its result (and to a matrix
instruction reading it as an A or B operand): the hardware does not hold
those back, so the result must be complete, which takes a number of
instruction slots that grows with the instruction's passes. The compiler
inserts the padding itself, but it has been seen to leave too little where
the consumer sits behind a branch, and the data read is then the
accumulator's previous value. The bound is the instruction's passes plus
four slots, the padding the compiler itself leaves in straight-line code; a
load may still overwrite a matrix result sooner, as its data returns long
after the result is written.
"""
from __future__ import annotations

import re
import subprocess
import tempfile
from dataclasses import dataclass, field
from pathlib import Path

from . import build as _build

_REG = re.compile(r"\b([va])(?:(\d+)\b|\[(\d+):(\d+)\])")
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_FUNC = re.compile(r"^(_Z\w+):")
_CAP = 64


def device_asm(src: Path) -> str:
    """gfx950 assembly of one source, built with the library's own flags."""
    src = Path(src)
    with tempfile.TemporaryDirectory() as td:
        out = Path(td) / (src.stem + ".s")
        cmd = [_build.HIPCC, *_build.COMMON, *_build.EXTRA.get(src.name, []), "--cuda-device-only", "-S",
               str(src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src.name}:\n{r.stderr}")
        return out.read_text()


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(2) is not None:
            out.add((kind, int(m.group(2))))
        else:
            for i in range(int(m.group(3)), int(m.group(4)) + 1):
                out.add((kind, i))
    return out


@dataclass
class _Insn:
    line: int
    op: str
    args: str
    asm: bool = False  # written as inline assembly (the compiler does not know its effects)


@dataclass
class _Block:
    label: str
    insns: list = field(default_factory=list)
    succ: list = field(default_factory=list)


def _functions(asm: str):
    """(name, [(line number, text)]) for every kernel body in the file."""
    name, body = None, []
    for no, raw in enumerate(asm.splitlines(), 1):
        m = _FUNC.match(raw)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if raw.startswith(".Lfunc_end"):
            yield name, body
            name = None
            continue
        body.append((no, raw))


def _blocks(body):
    blocks, cur = [], _Block("<entry>")
    blocks.append(cur)
    ends = False  # the current block ended with an unconditional branch or the program end

    def new(label):
        nonlocal cur
        nb = _Block(label)
        blocks.append(nb)
        cur = nb

    in_asm = False
    for no, raw in body:
        if ";;#ASMSTART" in raw:
            in_asm = True
            continue
        if ";;#ASMEND" in raw:
            in_asm = False
            continue
        m = _LABEL.match(raw)
        if m:
            prev = cur
            new(m.group(1))
            if not ends:
                prev.succ.append((None, cur.label))
            ends = False
            continue
        text = raw.split(";", 1)[0].strip()
        if not text or text.startswith("."):
            continue
        parts = text.split(None, 1)
        op, args = parts[0], parts[1] if len(parts) > 1 else ""
        if ends:  # code after an unconditional end starts a block of its own
            new(f"<after {no}>")
            ends = False
        cur.insns.append(_Insn(no, op, args, in_asm))
        if op == "s_branch":
            cur.succ.append((None, args.strip()))
            ends = True
        elif op.startswith("s_cbranch_"):
            cond = op[len("s_cbranch_"):]
            cur.succ.append((cond, args.strip()))
            prev = cur
            new(f"<fall {no}>")
            prev.succ.append(("not " + cond, cur.label))
        elif op in ("s_endpgm", "s_setpc_b64", "s_trap"):
            ends = True
    return blocks


def _lgkm_wait(args: str):
    m = re.search(r"lgkmcnt\((\d+)\)", args)
    return int(m.group(1)) if m else None


def _is_lds(op: str) -> bool:
    return op.startswith("ds_")


def _lds_dest(op: str, args: str) -> set:
    if op.startswith(("ds_read", "ds_load")) or "_rtn" in op or op in (
            "ds_bpermute_b32", "ds_permute_b32", "ds_swizzle_b32", "ds_append", "ds_consume"):
        first = args.split(",", 1)[0]
        return _regs(first)
    return set()


_SPAIR = re.compile(r"^s\[(\d+):(\d+)\]$")
_SREG = re.compile(r"\bs(?:(\d+)\b|\[(\d+):(\d+)\])")


def _sregs(text: str) -> set:
    out = set()
    for m in _SREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _env_step(env: dict, insn: _Insn) -> dict:
    """Known values of the lane-mask flags the structurizer branches on: an
    SGPR pair set to all-ones or zero, and vcc computed from one of them with
    exec (which is never zero where code runs)."""
    ops = [o.strip() for o in insn.args.split(",")] if insn.args else []
    dst = ops[0] if ops else ""
    out = dict(env)
    if insn.op == "s_mov_b64" and _SPAIR.match(dst) and len(ops) == 2 and ops[1] in ("-1", "0"):
        lo = int(_SPAIR.match(dst).group(1))
        for k in [k for k in out if k != "vcc" and (k[0] <= lo + 1 and lo <= k[1])]:
            del out[k]
        out[(lo, lo + 1)] = int(ops[1])
        return out
    if insn.op in ("s_andn2_b64", "s_and_b64") and dst == "vcc" and len(ops) == 3 and "exec" in ops[1:]:
        other = ops[2] if ops[1] == "exec" else ops[1]
        m = _SPAIR.match(other)
        key = (int(m.group(1)), int(m.group(2))) if m else None
        out.pop("vcc", None)
        if key in out:
            val = out[key]
            out["vcc"] = (val == 0) if insn.op == "s_andn2_b64" else (val == -1)  # vcc != 0
        return out
    written = _sregs(dst)
    if written:
        for k in [k for k in out if k != "vcc" and any(k[0] <= r <= k[1] for r in written)]:
            del out[k]
    if dst.startswith("vcc") or insn.op.endswith("_e32") and (
            insn.op.startswith("v_cmp") or "_co_" in insn.op or insn.op.startswith(("v_addc", "v_subb"))):
        out.pop("vcc", None)
    if insn.op.startswith("v_cmpx") or "exec" in dst:
        pass  # exec itself is not tracked
    return out


def _feasible(cond, env: dict) -> bool:
    if cond is None or "vcc" not in env:
        return True
    neg = cond.startswith("not ")
    c = cond[4:] if neg else cond
    if c not in ("vccnz", "vccz"):
        return True
    taken = env["vcc"] if c == "vccnz" else not env["vcc"]
    return taken != neg


def _mfma_slots(op: str) -> int:
    """Instruction slots a non-matrix reader must stay behind a matrix write:
    the instruction's passes (four cycles each on gfx950) plus four."""
    if "16x16x32" in op:
        passes = 4
    elif "32x32x16" in op or "16x16x128" in op:
        passes = 8
    else:
        passes = 16
    return passes + 4


def _wait_states(insn: _Insn) -> int:
    if insn.op == "s_nop":
        try:
            return int(insn.args.strip(), 0) + 1
        except ValueError:
            return 1
    return 1


def _step_mfma(state: dict, insn: _Insn, hazards: list | None, fname: str):
    """Transfer one instruction: state maps a register to (slots still owed, line of its matrix write)."""
    if insn.op in ("s_swappc_b64", "s_call_b64"):
        state.clear()  # the call and the callee's prologue are far more than any padding
        return
    if state and hazards is not None:
        if insn.op.startswith("v_mfma"):
            ops = [o.strip() for o in insn.args.split(",")]
            touched = _regs(",".join(ops[1:3])) if len(ops) >= 3 else set()
        elif insn.op.startswith(("ds_read", "ds_load", "buffer_load", "global_load", "scratch_load")):
            touched = _regs(insn.args.split(",", 1)[1]) if "," in insn.args else set()
        else:
            touched = _regs(insn.args)
        for r in sorted(touched & state.keys()):
            owed, line = state[r]
            hazards.append(f"{fname}: line {insn.line} `{insn.op} {insn.args}` uses {r[0]}{r[1]} "
                           f"{owed} slot(s) too soon after the matrix write at line {line}")
            break
    ws = _wait_states(insn)
    for r in list(state):
        owed, line = state[r]
        if owed - ws > 0:
            state[r] = (owed - ws, line)
        else:
            del state[r]
    if insn.op.startswith("v_mfma"):
        dst = insn.args.split(",", 1)[0]
        for r in _regs(dst):
            state[r] = (_mfma_slots(insn.op), insn.line)


def _merge_mfma(a: dict, b: dict) -> dict:
    out = dict(a)
    for r, v in b.items():
        if r not in out or v[0] > out[r][0]:
            out[r] = v
    return out


def _step(state: dict, insn: _Insn, hazards: list | None, fname: str):
    """Transfer one instruction: state maps line -> (later LDS ops, dest regs).
    Only reads written as inline assembly are tracked (the compiler waits for
    its own), but every LDS operation counts toward the later ones. A call
    waits for everything: a callee starts with a full s_waitcnt."""
    if insn.op in ("s_swappc_b64", "s_call_b64"):
        state.clear()
        return
    if insn.op == "s_waitcnt":
        n = _lgkm_wait(insn.args)
        if n is not None:
            for k in [k for k, (later, _) in state.items() if later >= n]:
                del state[k]
        return
    touched = _regs(insn.args)
    lds = _is_lds(insn.op)
    dest = _lds_dest(insn.op, insn.args) if lds else set()
    if hazards is not None and touched:
        for k, (later, regs) in state.items():
            clash = (touched - dest) & regs if lds else touched & regs
            if clash:
                r = sorted(clash)[0]
                hazards.append(f"{fname}: line {insn.line} `{insn.op} {insn.args}` touches "
                               f"{r[0]}{r[1]} before the LDS read at line {k} has returned")
                break
    if lds:
        for k in list(state):
            later, regs = state[k]
            regs = regs - dest  # an LDS write-after-write lands in order
            if regs:
                state[k] = (min(later + 1, _CAP), regs)
            else:
                del state[k]
        if dest and insn.asm:
            state[insn.line] = (0, dest)


def _merge(a: dict, b: dict) -> dict:
    out = dict(a)
    for k, (later, regs) in b.items():
        if k in out:
            out[k] = (min(out[k][0], later), out[k][1] | regs)
        else:
            out[k] = (later, regs)
    return out


def _key(env: dict):
    return tuple(sorted(env.items(), key=repr))


def check_function(fname: str, body) -> list:
    """Hazards of one kernel. The state at a block entry is a set of
    disjuncts, one per combination of known branch flags, each with its own
    pending LDS reads and matrix results, so the structurizer's flag-guarded
    paths that cannot both be taken are not merged."""
    blocks = _blocks(body)
    by_label = {b.label: b for b in blocks}
    entry = {b.label: {} for b in blocks}
    entry[blocks[0].label] = {_key({}): ({}, {}, {})}
    work = [blocks[0].label]
    while work:
        lab = work.pop()
        for env0, pend0, mf0 in list(entry[lab].values()):
            env, st, mf = dict(env0), dict(pend0), dict(mf0)
            for insn in by_label[lab].insns:
                _step(st, insn, None, fname)
                _step_mfma(mf, insn, None, fname)
                env = _env_step(env, insn)
            for cond, s in by_label[lab].succ:
                if s not in by_label or not _feasible(cond, env):
                    continue
                k = _key(env)
                old = entry[s].get(k)
                new = (env, st, mf) if old is None else (env, _merge(old[1], st), _merge_mfma(old[2], mf))
                if old is None or new[1] != old[1] or new[2] != old[2]:
                    entry[s][k] = new
                    if s not in work:
                        work.append(s)
    hazards = []
    for b in blocks:
        for env0, pend0, mf0 in entry[b.label].values():
            st, mf = dict(pend0), dict(mf0)
            for insn in b.insns:
                _step(st, insn, hazards, fname)
                _step_mfma(mf, insn, hazards, fname)
    return sorted(set(hazards))


def check_asm(asm: str) -> list:
    """Every use of a register an LDS read may still be writing, and every
    read of a matrix result too soon after its write, in every kernel."""
    out = []
    for name, body in _functions(asm):
        out.extend(check_function(name, body))
    return out


def checked_sources() -> list:
    """The sources that define kernels which wait for inline-assembly LDS
    reads by count or use matrix instructions (host-only sources that merely
    name such a launcher are left out: their device code holds no kernel)."""
    out = []
    for s in _build.sources():
        t = s.read_text()
        if "__global__" in t and ("lgkm_wait" in t or "mfma" in t):
            out.append(s)
    return out
