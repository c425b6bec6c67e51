"""Static check of the hand-issued memory instructions in the device assembly.

The grouped-query decode kernels issue their K loads (into registers) and
their transposed LDS reads with inline assembly, so that the waits before the
math can count exactly.  The compiler cannot see that such a load writes its
destination registers only when the data returns: if it regarded the result
as unused, or moved it to other registers before the wait, it could hand the
registers to another value while the load is still in flight, and the late
return would overwrite that value (an address, say).  This module proves, on
the generated assembly, that this never happens: for every inline-asm vector
memory load or LDS read with a VGPR destination, no instruction on any
control-flow path touches those registers until an ``s_waitcnt`` retires the
load.

Retirement: vector-memory operations return in issue order, so
``s_waitcnt vmcnt(N)`` retires a load once at least N vector-memory
operations were issued after it; an LDS read is retired by ``lgkmcnt(0)``.
The analysis is a forward dataflow over the basic blocks of each kernel; at a
join, a load stays pending if it is pending on any incoming path, with the
smallest count of younger operations.
"""
from __future__ import annotations

import re
from collections import defaultdict

_VMEM = re.compile(r'^(global_|buffer_|flat_|scratch_)')
_REG = re.compile(r'\bv\[(\d+):(\d+)\]|\bv(\d+)\b')
_DST = re.compile(r'^\S+\s+(v\[\d+:\d+\]|v\d+)')
_AGE_CAP = 64


def _regs(text: str) -> set[int]:
    out: set[int] = set()
    for a, b, c in _REG.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _blocks(lines: list[str]):
    """Basic blocks [(label, [(instruction, from_inline_asm)])] and successors."""
    blocks, cur, in_asm = [], ['<entry>', []], False
    for raw in lines:
        t = raw.strip()
        if t == ';;#ASMSTART':
            in_asm = True
            continue
        if t == ';;#ASMEND':
            in_asm = False
            continue
        if not t or t.startswith(';'):
            continue
        m = re.match(r'^(\.LBB\d+_\d+):', t)
        if m:
            blocks.append(cur)
            cur = [m.group(1), []]
            continue
        if t.startswith('.') or t.endswith(':'):
            continue
        t = t.split(';')[0].strip()
        cur[1].append((t, in_asm))
        if re.match(r's_(branch|cbranch_\w+|endpgm|setpc)\b', t):
            blocks.append(cur)
            cur = [f'<after {len(blocks)}>', []]
    blocks.append(cur)
    blocks = [b for b in blocks if b[1] or b[0].startswith('.LBB')]
    index = {b[0]: i for i, b in enumerate(blocks)}
    succ = defaultdict(list)
    for i, (_, ins) in enumerate(blocks):
        last = ins[-1][0] if ins else ''
        m = re.match(r's_(branch|cbranch_\w+)\s+(\.LBB\d+_\d+)', last)
        if m:
            succ[i].append(index[m.group(2)])
            if m.group(1) != 'branch' and i + 1 < len(blocks):
                succ[i].append(i + 1)
        elif not (last.startswith('s_endpgm') or last.startswith('s_setpc')) and i + 1 < len(blocks):
            succ[i].append(i + 1)
    return blocks, succ


def check_kernel(lines: list[str]) -> list[tuple[str, str, str]]:
    """Violations (pending load, offending instruction, block) in one kernel."""
    blocks, succ = _blocks(lines)
    problems: set[tuple[str, str, str]] = set()

    def transfer(i, state, report):
        st = dict(state)   # (kind, site) -> (registers, younger vm ops)
        for text, asm in blocks[i][1]:
            op = text.split()[0]
            if op == 's_waitcnt':
                m = re.search(r'vmcnt\((\d+)\)', text)
                if m:
                    n = int(m.group(1))
                    st = {k: v for k, v in st.items() if not (k[0] == 'vm' and v[1] >= n)}
                if 'lgkmcnt(0)' in text:
                    st = {k: v for k, v in st.items() if k[0] != 'ds'}
                continue
            touched = _regs(text)
            if report:
                for key, (regs, _) in st.items():
                    if touched & regs:
                        problems.add((key[1], text, blocks[i][0]))
            if _VMEM.match(text):
                st = {k: ((v[0], min(_AGE_CAP, v[1] + 1)) if k[0] == 'vm' else v) for k, v in st.items()}
                if asm and '_lds_' not in text and 'store' not in text:
                    m = _DST.match(text)
                    if m:
                        st[('vm', f'{blocks[i][0]}: {text}')] = (frozenset(_regs(m.group(1))), 0)
            elif asm and op.startswith('ds_read'):
                m = _DST.match(text)
                if m:
                    st[('ds', f'{blocks[i][0]}: {text}')] = (frozenset(_regs(m.group(1))), 0)
        return st

    state_in = {0: {}}
    work = [0]
    while work:
        i = work.pop()
        out = transfer(i, state_in[i], False)
        for s in succ[i]:
            old = state_in.get(s)
            new = dict(old) if old is not None else {}
            changed = old is None
            for k, v in out.items():
                if k not in new or v[1] < new[k][1]:
                    new[k] = v
                    changed = True
            if changed:
                state_in[s] = new
                work.append(s)
    for i in state_in:
        transfer(i, state_in[i], True)
    return sorted(problems)


def kernels(asm_text: str):
    """(symbol, lines) of every kernel body in an assembly file."""
    name, body = None, []
    for raw in asm_text.split('\n'):
        m = re.match(r'^(_Z\S+):\s*(;.*)?$', raw)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            if raw.strip().startswith('.Lfunc_end'):
                yield name, body
                name, body = None, []
            else:
                body.append(raw)


def check_assembly(asm_text: str) -> dict[str, list]:
    """Violations per kernel that contains inline assembly."""
    out = {}
    for name, body in kernels(asm_text):
        if any('ASMSTART' in l for l in body):
            out[name] = check_kernel(body)
    return out
