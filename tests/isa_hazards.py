"""Static check of matrix-core data hazards in a gfx950 assembly listing.

The prefill GEMM issues its MFMAs through inline assembly, which the
compiler's hazard recognizer does not see, so the required independent
instructions between an MFMA and its neighbours must come from the source.
This walks the control-flow graph of one kernel in the listing and checks:

  R1  a VALU write of a register (VGPR or AGPR) followed by an MFMA that
      reads it (A, B or C operand) needs at least `valu_mfma` wait states;
  R2  an MFMA result followed by any non-MFMA instruction that reads or
      writes those registers needs at least `mfma_other` wait states.

Wait states are counted one per instruction, s_nop N as N + 1; every path
through branches is followed.  The limits used by the test are above the
largest values for these cases in the CDNA3/CDNA4 instruction-set manuals'
dependency tables (VALU write -> MFMA read: 2; 4-pass XDL write -> VALU
access: at most 11 on gfx950), so a pass is conservative.
"""
import re

_REG = re.compile(r'^([va])\[(\d+):(\d+)\]$|^([va])(\d+)$')


def _regs(tok):
    m = _REG.match(tok.strip())
    if not m:
        return frozenset()
    if m.group(1):
        return frozenset((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset([(m.group(4), int(m.group(5)))])


def parse_kernel(text, symbol):
    """Instructions of `symbol` as (opcode, operands) with label/branch maps."""
    insts, labels = [], {}
    on = False
    for line in text.splitlines():
        if not on:
            if line.startswith(symbol + ':'):
                on = True
            continue
        body = line.split(';')[0].strip()
        if not body:
            continue
        if body.endswith(':'):
            labels[body[:-1]] = len(insts)
            continue
        if body.startswith('.'):
            continue
        parts = body.split(None, 1)
        ops = [o.strip() for o in parts[1].split(',')] if len(parts) > 1 else []
        insts.append((parts[0], ops))
        if parts[0] == 's_endpgm':
            break
    if not insts:
        raise ValueError('kernel %s not found' % symbol)
    return insts, labels


def _cfg(insts, labels):
    succ = [[] for _ in insts]
    for k, (op, ops) in enumerate(insts):
        if op.startswith('s_cbranch') or op == 's_branch':
            tgt = labels.get(ops[0]) if ops else None
            if tgt is not None:
                succ[k].append(tgt)
            if op.startswith('s_cbranch') and k + 1 < len(insts):
                succ[k].append(k + 1)
        elif op != 's_endpgm' and k + 1 < len(insts):
            succ[k].append(k + 1)
    pred = [[] for _ in insts]
    for k, ss in enumerate(succ):
        for s in ss:
            pred[s].append(k)
    return succ, pred


def _cost(inst):
    op, ops = inst
    if op == 's_nop':
        return int(ops[0], 0) + 1
    return 1


def check(text, symbol, valu_mfma=4, mfma_other=19):
    insts, labels = parse_kernel(text, symbol)
    succ, pred = _cfg(insts, labels)
    found = []

    def is_mfma(op):
        return op.startswith('v_mfma')

    for k, (op, ops) in enumerate(insts):
        if not is_mfma(op):
            continue
        reads = frozenset().union(*(_regs(o) for o in ops[1:4]))
        # R1: walk predecessors while fewer than valu_mfma wait states separate them
        stack = [(p, 0) for p in pred[k]]
        seen = set()
        while stack:
            j, dist = stack.pop()
            if (j, dist) in seen or dist >= valu_mfma:
                continue
            seen.add((j, dist))
            op2, ops2 = insts[j]
            if op2.startswith('v_') and not is_mfma(op2) and ops2 and (_regs(ops2[0]) & reads):
                found.append(('R1', dist, insts[j], insts[k]))
                continue
            stack.extend((p, dist + _cost(insts[j])) for p in pred[j])
        # R2: walk successors
        dst = _regs(ops[0])
        stack = [(s, 0) for s in succ[k]]
        seen = set()
        while stack:
            j, dist = stack.pop()
            if (j, dist) in seen or dist >= mfma_other:
                continue
            seen.add((j, dist))
            op2, ops2 = insts[j]
            if not is_mfma(op2) and any(_regs(o) & dst for o in ops2):
                found.append(('R2', dist, insts[k], insts[j]))
                continue
            stack.extend((s, dist + _cost(insts[j])) for s in succ[j])
    n_mfma = sum(1 for op, _ in insts if is_mfma(op))
    return n_mfma, found
