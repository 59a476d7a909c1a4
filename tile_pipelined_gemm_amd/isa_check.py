"""Build-time checks of the gfx950 assembly of every kernel: no loop that
holds a workgroup barrier may be left on an exec-mask branch, no register
spill may sit among the MFMAs of a K loop, no 12/16-byte buffer store may
have its data registers rewritten right after it, and no LDS DMA may follow
a scalar write of M0 without a wait state between them.

A persistent kernel's role loops contain s_barrier and end in a
`if (threadIdx.x == 0) { ... }` block (queue atomics, releases).  When the
compiler cannot prove a loop's exit uniform it may lower the loop with a
per-lane exit (the lanes of a wave leave one by one, under exec masks) and
move such a block onto the exit path.  The waves then keep executing the
barriers without the work that block does for them: the kernel spins for
ever.  Uniform exits (scalar branches on values made wave-uniform with
readfirstlane) never take that form, so the check is structural: in the
control-flow graph of each kernel, a strongly connected region that
contains s_barrier must not have an s_cbranch_execz/execnz edge leading out
of it.
"""
import re
import sys

_BRANCH = re.compile(r"(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)")


def kernels(asm_text):
    """Yield (symbol, [instruction lines]) for each function in the file."""
    name, body = None, []
    for ln in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        body.append(ln)
        if "s_endpgm" in ln:
            yield name, body
            name, body = None, []


def _blocks(lines):
    """Split into basic blocks: (label or None, [instructions])."""
    out, cur, lab = [], [], ".entry"
    for raw in lines:
        m = re.match(r"^(\.LBB\w+):", raw)
        if m:
            if cur or lab:
                out.append((lab, cur))
            lab, cur = m.group(1), []
            continue
        ins = raw.split(";")[0].strip()
        if not ins or ins.startswith("."):
            continue
        cur.append(ins)
        if _BRANCH.match(ins) or ins.startswith("s_endpgm") or ins.startswith("s_setpc"):
            out.append((lab, cur))
            lab, cur = None, []
    if cur:
        out.append((lab, cur))
    return out


def divergent_barrier_loops(lines):
    """Return [(block label, branch)] for exec-mask exits of barrier loops."""
    bl = _blocks(lines)
    index_of = {lab: i for i, (lab, _) in enumerate(bl) if lab}
    succ, exec_branch = [], []
    for i, (_, ins) in enumerate(bl):
        s, eb = [], False
        last = ins[-1] if ins else ""
        m = _BRANCH.match(last)
        if m:
            if m.group(2) in index_of:
                s.append(index_of[m.group(2)])
            if m.group(1) != "s_branch" and i + 1 < len(bl):
                s.append(i + 1)
            eb = m.group(1) in ("s_cbranch_execz", "s_cbranch_execnz")
        elif not last.startswith("s_endpgm") and i + 1 < len(bl):
            s.append(i + 1)
        succ.append(s)
        exec_branch.append(eb)

    # strongly connected components (iterative Tarjan)
    n = len(bl)
    index, low, on_stack, stack, comp = [-1] * n, [0] * n, [False] * n, [], [-1] * n
    counter = 0
    for root in range(n):
        if index[root] >= 0:
            continue
        work = [(root, 0)]
        while work:
            v, k = work.pop()
            if k == 0:
                index[v] = low[v] = counter
                counter += 1
                stack.append(v)
                on_stack[v] = True
            if k < len(succ[v]):
                work.append((v, k + 1))
                w = succ[v][k]
                if index[w] < 0:
                    work.append((w, 0))
                elif on_stack[w]:
                    low[v] = min(low[v], index[w])
                continue
            for w in succ[v]:
                if on_stack[w] and comp[w] < 0:
                    low[v] = min(low[v], low[w])
            if low[v] == index[v]:
                while True:
                    w = stack.pop()
                    on_stack[w] = False
                    comp[w] = v
                    if w == v:
                        break
    groups = {}
    for v in range(n):
        groups.setdefault(comp[v], []).append(v)
    bad = []
    for members in groups.values():
        ms = set(members)
        if len(members) == 1 and members[0] not in succ[members[0]]:
            continue                                   # not a loop
        if not any(ins.startswith("s_barrier") for v in members for ins in bl[v][1]):
            continue
        for v in members:
            if exec_branch[v] and any(w not in ms for w in succ[v]):
                bad.append((bl[v][0], bl[v][1][-1]))
    return bad


def spills_among_mfma(lines, window=8):
    """Return the scratch (register spill) instructions that sit between matrix
    instructions -- within `window` instructions of an MFMA on both sides,
    i.e. inside an MFMA loop body, where a spill costs a memory round trip
    per K step."""
    ins = [ln.split(";")[0].strip() for ln in lines]
    ins = [x for x in ins if x and not x.startswith(".") and not x.endswith(":")]
    mf = [i for i, x in enumerate(ins) if x.startswith("v_mfma")]
    bad = []
    for i, x in enumerate(ins):
        if not x.startswith("scratch_"):
            continue
        before = any(i - window <= j < i for j in mf)
        after = any(i < j <= i + window for j in mf)
        if before and after:
            bad.append(x)
    return bad


_STORE_WIDE = re.compile(r"^buffer_store_dwordx[34]\s+v\[(\d+):(\d+)\]")
_VDST = re.compile(r"^v_\w+\s+(?:v(\d+)|v\[(\d+):(\d+)\])")


def wide_store_data_overwrites(lines, wait_states=2):
    """Return the 12/16-byte buffer stores whose data registers an ALU
    instruction rewrites within `wait_states` wait states.  Such a store can
    read its data late enough to pick up the new value (observed on gfx950),
    and the compiler inserts no wait for buffer stores with a register
    soffset, so the code must not produce the pattern."""
    ins = [ln.split(";")[0].strip() for ln in lines]
    ins = [x for x in ins if x and not x.startswith(".") and not x.endswith(":")]
    bad = []
    for i, x in enumerate(ins):
        m = _STORE_WIDE.match(x)
        if not m:
            continue
        lo, hi = int(m.group(1)), int(m.group(2))
        ws, j = 0, i + 1
        while ws < wait_states and j < len(ins):
            y = ins[j]
            d = _VDST.match(y)
            if d:
                a = int(d.group(1) or d.group(2))
                b = int(d.group(1) or d.group(3))
                if a <= hi and b >= lo:
                    bad.append(f"{x} | {y}")
                    break
            n = re.match(r"^s_nop\s+(\d+)", y)
            ws += int(n.group(1)) + 1 if n else 1
            j += 1
    return bad


_M0_WRITE = re.compile(r"^s_\w+\s+m0\s*,")
_LDS_DMA = re.compile(r"^(buffer|global)_load_\w+\s.*\blds\b")


def m0_lds_dma_hazards(lines):
    """Return the LDS DMA loads (buffer/global loads with the lds bit) that
    come directly after a scalar instruction writing M0.  On gfx9-family parts
    the DMA reads M0 (its LDS address) one wait state after such a write: with
    no instruction or s_nop in between it can use the old value and fill the
    wrong LDS slot.  The compiler's hazard recognizer inserts the s_nop for
    the loads it emits, but not inside inline asm."""
    ins = [ln.split(";")[0].strip() for ln in lines]
    ins = [x for x in ins if x and not x.startswith(".") and not x.endswith(":")]
    return [f"{a} | {b}" for a, b in zip(ins, ins[1:]) if _M0_WRITE.match(a) and _LDS_DMA.match(b)]


def check_file(path):
    """Return {kernel symbol: findings} for kernels with findings."""
    with open(path) as f:
        text = f.read()
    found = {}
    for name, lines in kernels(text):
        b = divergent_barrier_loops(lines)
        sp = spills_among_mfma(lines)
        if sp:
            b = b + [("spill among MFMAs", x) for x in sp[:3]]
        ow = wide_store_data_overwrites(lines)
        if ow:
            b = b + [("store data rewritten", x) for x in ow[:3]]
        m0 = m0_lds_dma_hazards(lines)
        if m0:
            b = b + [("LDS DMA right after an M0 write", x) for x in m0[:3]]
        if b:
            found[name] = b
    return found


if __name__ == "__main__":
    rc = 0
    for p in sys.argv[1:]:
        for k, v in check_file(p).items():
            print(f"{p}: {k}: {v[:3]}")
            rc = 1
    sys.exit(rc)
