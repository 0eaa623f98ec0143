"""Build-time check of the gfx950 assembly of kernels that issue their own
vector loads.

The big-tile GEMM issues its global loads as inline asm and waits for them
with explicit `s_waitcnt vmcnt(N)`, so the compiler does not know that the
destination registers of those loads are still being written.  This check
walks every kernel's control-flow graph and proves, for every path, that no
instruction reads or writes a register of a load that the waits have not yet
retired (loads retire in order: `vmcnt(N)` retires all but the newest N).
It also rejects scratch (spill) traffic, which would add loads the waits do
not count, and any scalar-memory store, write-back or atomic.

Usage: python -m mixture_experts_expert_moe_amd.asm_check file.s [kernel-substring]
"""
from __future__ import annotations

import re
import sys

_FORBIDDEN = re.compile(r"^\s*(s_store|s_buffer_store|s_atomic|s_buffer_atomic|s_dcache_wb|scratch_load|scratch_store)")


def _vregs(tok: str) -> frozenset:
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _kernel_bodies(asm: str, pattern: str):
    for name in re.findall(r"^(_Z\S*%s\S*):" % re.escape(pattern), asm, re.M):
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        lines = [l.split(";")[0].strip() for l in body.splitlines()[1:]]
        yield name, [l for l in lines if l and (not l.startswith(".") or re.match(r"\.LBB\S+:$", l))]


def check_kernel(text: list) -> list:
    """Return a list of (instruction index, text, offending pending load) for one kernel."""
    labels = {l[:-1]: i for i, l in enumerate(text) if l.endswith(":")}

    def successors(i):
        l = text[i]
        if l.split(" ")[0] == "s_endpgm":
            return []
        m = re.match(r"s_(cbranch_\w+|branch)\s+(\.LBB\S+)", l)
        out = []
        if m:
            out.append(labels[m.group(2)])
            if m.group(1) == "branch":
                return out
        if i + 1 < len(text):
            out.append(i + 1)
        return out

    def is_lds_dma(op, rest):
        return op.startswith(("global_load_lds", "buffer_load_lds")) or " lds" in rest

    bad = set()

    def transfer(i, st):
        l = text[i]
        if l.endswith(":"):
            return st
        op, _, rest = l.partition(" ")
        ops = rest.split(",")
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", rest)
            if m:
                n = int(m.group(1))
                st = {k: c for k, c in st.items() if c < n}
            return st
        is_load = op.startswith(("global_load", "buffer_load", "scratch_load"))
        dma = is_lds_dma(op, rest)
        used = frozenset()
        for t in (ops[1:] if is_load and not dma else ops):
            used |= _vregs(t)
        for k in st:
            kop, _, krest = text[k].partition(" ")
            if is_lds_dma(kop, krest):
                continue  # data goes to LDS: no register destination
            if used & _vregs(krest.split(",")[0]):
                bad.add((i, k))
        if is_load or op.startswith(("global_store", "buffer_store", "global_atomic", "scratch_store")):
            st = {k: min(c + 1, 64) for k, c in st.items()}
            if is_load:
                st[i] = 0
        return st

    # forward dataflow: for every load still pending, the least number of loads issued after it
    state = {0: {}}
    work = [0]
    while work:
        i = work.pop()
        out = transfer(i, state[i])
        for j in successors(i):
            old = state.get(j)
            if old is None:
                new = dict(out)
            else:
                new = dict(old)
                for k, c in out.items():
                    new[k] = min(c, new.get(k, 99))
            if new != old:
                state[j] = new
                work.append(j)
    return [(i, text[i], text[k]) for i, k in sorted(bad)]


def check_file(path: str, pattern: str = "big_gemm_kernel") -> list:
    asm = open(path).read()
    problems = []
    found = 0
    for name, text in _kernel_bodies(asm, pattern):
        found += 1
        for i, l, k in check_kernel(text)[:5]:
            problems.append("%s: instruction %d '%s' touches a register of the pending load '%s'" % (name, i, l, k))
        for l in text:
            if _FORBIDDEN.match(l):
                problems.append("%s: forbidden instruction '%s'" % (name, l))
                break
    if not found:
        problems.append("no kernel matching %r in %s" % (pattern, path))
    return problems


if __name__ == "__main__":
    probs = check_file(sys.argv[1], *(sys.argv[2:3]))
    for p in probs:
        print(p)
    sys.exit(1 if probs else 0)
