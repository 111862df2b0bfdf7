"""Static check of matrix-core result reads in gfx950 assembly.

A VALU instruction (or a store) that reads a register an MFMA writes must
come a number of wait states after that MFMA; the hardware does not hold it
back, and a read that comes too early returns the register's old value.
The numbers below were measured on the MI355X with one wave that issues an
MFMA, a given number of s_nop wait states, then a read of its last result
register (tests/mfma_wait_probe.hip; tests/test_mfma_wait_states_gpu.py runs
it again): with fewer, the read returns the old value.

The compiler inserts these wait states itself, but for the scaled fp8
product it allows 19 on some control-flow paths, one fewer than the
hardware needs.  check() walks every path of a compiled kernel from each
MFMA and reports reads that come too early.

prefetch_waits() looks for a performance fault of the same compiled code: a
memory-counter wait that holds the matrix cores until the LDS-DMA loads of
the next tile have landed.  A double-buffered tile loop queues those loads
and then computes on the tile loaded before; a wait placed between the two
(the compiler adds one when it cannot see that an earlier wait already
covered the loads the products read) turns the prefetch into a stall.
"""
import re

# wait states a VALU read of an MFMA's destination needs, measured on MI355X
WAIT_STATES = {
    "v_mfma_scale_f32_32x32x64_f8f6f4": 20,
    "v_mfma_f32_32x32x16_bf16": 12,
}

_STORE_PREFIXES = ("global_store", "buffer_store", "ds_write", "scratch_store", "flat_store")
_READ_PREFIXES = ("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")


def registers(token):
    """VGPR numbers named by one operand (v7, v[8:11]); empty for others."""
    token = token.strip().split()[0] if token.strip() else ""
    m = re.match(r"v\[(\d+):(\d+)\]$", token)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", token)
    return {int(m.group(1))} if m else set()


def _split(line):
    parts = line.split(None, 1)
    ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def parse_kernels(text):
    """{kernel symbol: (instructions, {label: index})} from an assembly file."""
    lines = text.splitlines()
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*:", l)]
    kernels = {}
    for n, a in enumerate(starts):
        name = lines[a].split(":")[0]
        end = starts[n + 1] if n + 1 < len(starts) else len(lines)
        ins, labels = [], {}
        for l in lines[a + 1:end]:
            if l.startswith(".Lfunc_end"):
                break
            l = l.split(";")[0].strip()
            if not l:
                continue
            m = re.match(r"^(\.LBB\S+|\d+):$", l)
            if m:
                labels[m.group(1)] = len(ins)
                continue
            if l.startswith(".") or l.endswith(":"):
                continue
            ins.append(l)
        if ins:
            kernels[name] = (ins, labels)
    return kernels


def _successors(i, ins, labels):
    op, ops = _split(ins[i])
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[ops[0]]]
    if op.startswith("s_cbranch"):
        return [labels[ops[0]], i + 1]
    return [i + 1] if i + 1 < len(ins) else []


def _reads(op, ops):
    if op.startswith("v_mfma"):
        # sources A and B and any scale operands; an accumulation into the
        # same registers (source C) is forwarded by the matrix core
        regs = set()
        for k, t in enumerate(ops[1:], start=1):
            if k != 3:
                regs |= registers(t)
        return regs
    if op.startswith("buffer_load") and ops and ops[-1].endswith("lds"):
        return registers(ops[0])
    if not op.startswith(_READ_PREFIXES):
        return set()
    start = 0 if op.startswith(_STORE_PREFIXES) else 1
    regs = set()
    for t in ops[start:]:
        regs |= registers(t)
    return regs


def _writes(op, ops):
    if op.startswith(_STORE_PREFIXES) or not op.startswith(("v_", "ds_read", "global_load", "buffer_load", "scratch_load", "flat_load")):
        return set()
    if op.startswith("buffer_load") and ops and ops[-1].endswith("lds"):
        return set()
    return registers(ops[0]) if ops else set()


def check(ins, labels):
    """Reads of an MFMA result with too few wait states, on any path:
    a list of (mfma index, read index, wait states)."""
    found = []
    for i, line in enumerate(ins):
        op, ops = _split(line)
        if not op.startswith("v_mfma"):
            continue
        if op not in WAIT_STATES:
            raise KeyError("no measured wait states for %s" % op)
        need = WAIT_STATES[op]
        stack = [(i + 1, 0, frozenset(registers(ops[0])))]
        seen = set()
        while stack:
            j, states, live = stack.pop()
            if states >= need or not live or j >= len(ins) or (j, states, live) in seen:
                continue
            seen.add((j, states, live))
            o, a = _split(ins[j])
            if o == "s_nop":
                nxt = states + int(a[0], 0) + 1
            else:
                nxt = states + 1
                if _reads(o, a) & live:
                    found.append((i, j, states))
                    continue
                live = live - _writes(o, a)
            for s in _successors(j, ins, labels):
                stack.append((s, nxt, live))
    return found


_VMEM_PREFIXES = ("buffer_", "global_", "scratch_", "flat_")


def prefetch_waits(ins, min_products=8):
    """Waits that force LDS-DMA loads queued since the last full memory wait
    to complete and are followed by at least `min_products` MFMAs before the
    next barrier, branch or end: a list of (wait index, products).

    The scan is linear.  On gfx9 every vector-memory instruction (loads,
    stores, scratch accesses) counts in vmcnt and completes in order, so
    s_waitcnt vmcnt(n) completes all but the last n of them.
    """
    found = []
    pending = []          # vector-memory ops since the last vmcnt(0): True = LDS DMA
    for i, line in enumerate(ins):
        op, ops = _split(line)
        if op.startswith(_VMEM_PREFIXES):
            pending.append(op.startswith("buffer_load") and bool(ops) and ops[-1].endswith("lds"))
            continue
        if op != "s_waitcnt":
            continue
        m = re.search(r"vmcnt\((\d+)\)", line)
        if not m:
            continue
        done = pending[:max(0, len(pending) - int(m.group(1)))]
        if any(done):
            products = 0
            for later in ins[i + 1:]:
                o = later.split()[0]
                if o in ("s_barrier", "s_branch", "s_endpgm") or o.startswith("s_cbranch"):
                    break
                if o.startswith("v_mfma"):
                    products += 1
            if products >= min_products:
                found.append((i, products))
        pending = pending[len(done):]
    return found
