"""Static check of hand-timed reads in the gfx950 device assembly.

Some kernels issue LDS reads (ds_read_*) and scalar loads (s_load_*) from
inline asm and wait for them themselves with `s_waitcnt lgkmcnt(N)`, so that
the reads of the next operands overlap the matrix-core work on the current
ones.  The compiler treats an inline-asm output as ready the moment the asm
statement ends: nothing stops the register allocator from copying such a
register, or reusing it, before the wait that makes it valid.  Such a copy
reads whatever the register held before the load lands, with no error.

This module walks every kernel's control-flow graph in the compiler's output
and reports any instruction that reads or writes a register whose inline-asm
load is still in flight.  The counting rules are the CDNA ones:

* LDS operations return in issue order, so `lgkmcnt(N)` retires every LDS
  read that has at least N younger LDS operations behind it (scalar loads in
  flight only lower the number of LDS reads still outstanding).
* Scalar memory loads can return in any order: only `lgkmcnt(0)` retires one.

The state at a join is the worst case over its predecessors (fewest younger
operations), iterated to a fixed point over loops.
"""
import os
import re
import subprocess

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_FUNC = re.compile(r"^([A-Za-z_.$][\w.$]*):[ \t]*;[ \t]*@\S+\n(.*?)^\.Lfunc_end", re.S | re.M)
_CAP = 16          # lgkmcnt is a 4-bit field on gfx9: ages at or above 16 are equivalent


def _regs(pat, text, tag):
    out = set()
    for m in pat.finditer(text):
        if m.group(3) is not None:
            out.add((tag, int(m.group(3))))
        else:
            out.update((tag, r) for r in range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _operands(text):
    return _regs(_VREG, text, "v") | _regs(_SREG, text, "s")


def _parse(lines):
    """-> list of (kind, text, from_inline_asm); kind is 'label' or 'ins'."""
    out, in_asm = [], False
    for raw in lines:
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = s.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":") and " " not in s:
            out.append(("label", s[:-1], in_asm))
        elif not s.startswith("."):
            out.append(("ins", s, in_asm))
    return out


def _join(a, b):
    if a is None:
        return dict(b)
    r = dict(a)
    for k, v in b.items():
        r[k] = min(v, r.get(k, _CAP))
    return r


def check_function(lines):
    """Hazards in one function's assembly lines -> sorted list of
    (index, instruction, reason).  The state maps a register to the number of
    LDS operations issued after the load that writes it ('s' registers of an
    asm scalar load carry -1: only lgkmcnt(0) retires them)."""
    ins = _parse(lines)
    label_at = {t: i for i, (k, t, _) in enumerate(ins) if k == "label"}
    entry = {0: {}}
    found = set()
    for _ in range(64):
        changed = False
        st = None
        for i, (kind, text, from_asm) in enumerate(ins):
            if i in entry:
                st = _join(st, entry[i]) if st is not None else dict(entry[i])
            if st is None:
                continue
            if kind == "label":
                merged = _join(entry.get(i), st)
                if merged != entry.get(i):
                    entry[i] = merged
                    changed = True
                st = dict(entry[i])
                continue
            op = text.split()[0]
            args = text[len(op):]
            if op.startswith("s_waitcnt"):
                m = _LGKM.search(args)
                n = int(m.group(1)) if m else (0 if args.strip() == "0" else None)
                if n is not None:
                    st = {r: a for r, a in st.items() if (a < n if a >= 0 else n != 0)}
                continue
            parts = args.split(",")
            dst, src = _operands(parts[0]), _operands(",".join(parts[1:]))
            touched = dst | src
            if from_asm and op.startswith("ds_read"):
                # LDS returns in order: a later read may target the register of
                # an earlier one still in flight; its address may not be in flight
                touched = src | {r for r in dst if st.get(r, 0) < 0}
            for r in touched & set(st):
                found.add((i, text, "%s%d touched while its asm load is in flight" % r))
            if op.startswith("ds_"):
                st = {r: (min(a + 1, _CAP) if a >= 0 else a) for r, a in st.items()}
                if from_asm and op.startswith("ds_read"):
                    for r in dst:
                        st[r] = 0
            elif from_asm and op.startswith("s_load"):
                for r in dst:
                    st[r] = -1
            if op == "s_branch" or op.startswith("s_cbranch"):
                target = args.strip().split()[-1]
                if target in label_at:
                    j = label_at[target]
                    merged = _join(entry.get(j), st)
                    if merged != entry.get(j):
                        entry[j] = merged
                        changed = True
                if op == "s_branch":
                    st = None
            elif op in ("s_endpgm", "s_setpc_b64"):
                st = None
        if not changed:
            break
    return sorted(found)


def check_asm(text):
    """-> list of (function, index, instruction, reason) over every function."""
    out = []
    for m in _FUNC.finditer(text):
        for i, ins, why in check_function(m.group(2).split("\n")):
            out.append((m.group(1), i, ins, why))
    return out


def device_asm(src, hipcc, flags):
    """gfx950 device assembly of one source, compiled with the build's flags."""
    cmd = [hipcc, *[f for f in flags if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("device asm failed: %s\n%s" % (" ".join(cmd), r.stderr))
    return r.stdout


def check_sources(csrc, sources, hipcc, flags):
    """Raise if any kernel of the given sources touches an in-flight asm load."""
    bad = []
    for s in sources:
        for fn, i, ins, why in check_asm(device_asm(os.path.join(csrc, s), hipcc, flags)):
            bad.append("%s: %s: [%d] %s -- %s" % (s, fn, i, ins, why))
    if bad:
        raise RuntimeError("in-flight asm loads touched before their wait:\n  " + "\n  ".join(bad[:40]))
