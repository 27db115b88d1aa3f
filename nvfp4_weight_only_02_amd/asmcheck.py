"""Static check of the gfx950 code built here: no instruction may read or write
a destination register of a vector-memory load that may still be in flight.

The GEMV and GEMM kernels issue their weight and activation loads as inline
assembly and wait for them with hand-counted ``s_waitcnt vmcnt(N)``; the
compiler sees such a load's destination as written when the asm statement
runs.  If it ever copied, reused or read one of those registers before the
wait that covers the load (for example across a branch it duplicated), the
result would be wrong data or, when the register holds an address, a fault.
Register spills are refused by the build; this check covers the rest, on the
disassembly of the built library.

The analysis is a forward dataflow over each kernel's control-flow graph.  The
state is the list of vector-memory operations that may be outstanding, newest
last, each with the registers it will write.  On gfx9, loads and stores both
count in vmcnt and complete in issue order, so ``s_waitcnt vmcnt(N)`` leaves
at most the N newest outstanding.  Where paths join, the states are aligned at
their newest entry and merged entry by entry (union of registers, the longer
length), which over-approximates every path.  Any instruction that names a
register of an outstanding load is reported.
"""
from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import tempfile

LLVM_BIN = "/opt/rocm/llvm/bin"
MAX_VMCNT = 63          # gfx9 vmcnt field: at most this many outstanding

_ADDR = re.compile(r"//\s*([0-9A-Fa-f]+):")
_FUNC = re.compile(r"^[0-9a-f]+ <([^>]+)>:\s*$")
_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_BRANCH = re.compile(r"^s_(c?branch)\w*$")


def llvm_tool(name: str) -> str:
    path = os.path.join(LLVM_BIN, name)
    if os.path.exists(path):
        return path
    found = shutil.which(name)
    if not found:
        raise RuntimeError("%s not found: cannot check the built code" % name)
    return found


def disassemble(lib: str, arch: str = "gfx950") -> str:
    """Disassembly of the `arch` code object bundled in the shared library `lib`."""
    objdump = llvm_tool("llvm-objdump")
    with tempfile.TemporaryDirectory() as tmp:
        copy = os.path.join(tmp, "lib.so")
        shutil.copyfile(lib, copy)
        subprocess.run([objdump, "--offloading", copy], cwd=tmp, check=True,
                       stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        objs = [f for f in os.listdir(tmp) if f.endswith("--" + arch)]
        if len(objs) != 1:
            raise RuntimeError("no single %s code object in %s (found %s)" % (arch, lib, objs))
        res = subprocess.run([objdump, "-d", "--mcpu=" + arch, os.path.join(tmp, objs[0])],
                             check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        return res.stdout


def parse(text: str) -> dict:
    """{function name: [(address, mnemonic, operand text), ...]} in address order."""
    funcs, cur = {}, None
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None or not line.startswith(("\t", " ")):
            continue
        a = _ADDR.search(line)
        if not a:
            continue
        body = line[:a.start()].strip()
        if not body:
            continue
        mnem, _, ops = body.partition(" ")
        cur.append((int(a.group(1), 16), mnem, ops.strip()))
    return funcs


def registers(ops: str) -> frozenset:
    """VGPRs and AGPRs named in an operand list, as ('v'|'a', index) pairs."""
    out = set()
    for kind, lo, hi, one in _REG.findall(ops):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return frozenset(out)


def is_vmem(mnem: str) -> bool:
    return mnem.startswith(("buffer_", "global_", "flat_", "scratch_"))


def vmem_dest(mnem: str, ops: str) -> frozenset:
    """Registers a vector-memory operation writes when it completes."""
    first = ops.split(",")[0].strip() if ops else ""
    words = ops.replace(",", " ").split()
    if "_load" in mnem:
        if "lds" in words:          # LDS-direct load: no register destination
            return frozenset()
        return registers(first)
    if "_atomic" in mnem and ("sc0" in words or "glc" in words):
        return registers(first)     # returning atomic
    return frozenset()              # store, non-returning atomic, cache operation


def vmcnt_of_waitcnt(ops: str):
    """The vmcnt a s_waitcnt waits for, or None if it does not wait on vmcnt."""
    m = re.search(r"vmcnt\((\d+)\)", ops)
    if m:
        return int(m.group(1))
    if re.fullmatch(r"(0x[0-9a-fA-F]+|\d+)", ops.strip()):
        v = int(ops.strip(), 0)     # gfx9 simm16: vmcnt = bits 3:0 | bits 15:14 << 4
        return (v & 0xF) | ((v >> 14) & 0x3) << 4
    return None


def branch_target(addr: int, ops: str) -> int:
    """Target of a SOPP branch: its 16-bit signed word offset from the next
    instruction (the disassembler prints it unsigned)."""
    v = int(ops.split()[0], 0) & 0xFFFF
    if v >= 0x8000:
        v -= 0x10000
    return addr + 4 + 4 * v


def merge(a: tuple, b: tuple) -> tuple:
    """Entry-wise union of two outstanding lists aligned at their newest entry."""
    n = max(len(a), len(b))
    out = []
    for k in range(n, 0, -1):
        x = a[-k] if k <= len(a) else frozenset()
        y = b[-k] if k <= len(b) else frozenset()
        out.append(x | y)
    return tuple(out)


def check_function(instrs: list, stats: dict = None) -> list:
    """Violations [(address, instruction text, registers)] of one function.
    If `stats` is given it receives the number of vector-memory operations
    seen and the longest outstanding list reached."""
    if not instrs:
        return []
    index = {a: i for i, (a, _, _) in enumerate(instrs)}
    for _, mnem, _ in instrs:
        if mnem in ("s_setpc_b64", "s_swappc_b64", "s_cbranch_join", "s_cbranch_g_fork", "s_cbranch_i_fork"):
            raise RuntimeError("indirect control flow (%s) is not analysed" % mnem)
    # Basic blocks: leaders are the entry, branch targets and what follows a
    # branch or s_endpgm.
    leaders = {0}
    for i, (addr, mnem, ops) in enumerate(instrs):
        if _BRANCH.match(mnem):
            t = branch_target(addr, ops)
            if t not in index:
                raise RuntimeError("branch at %#x to %#x outside the function" % (addr, t))
            leaders.add(index[t])
            if i + 1 < len(instrs):
                leaders.add(i + 1)
        elif mnem == "s_endpgm" and i + 1 < len(instrs):
            leaders.add(i + 1)
    starts = sorted(leaders)
    blocks = {s: (s, (starts[j + 1] if j + 1 < len(starts) else len(instrs))) for j, s in enumerate(starts)}
    succ = {}
    for s, (b, e) in blocks.items():
        addr, mnem, ops = instrs[e - 1]
        nxt = [e] if e < len(instrs) else []
        if mnem == "s_endpgm":
            succ[s] = []
        elif mnem == "s_branch":
            succ[s] = [index[branch_target(addr, ops)]]
        elif _BRANCH.match(mnem):
            succ[s] = [index[branch_target(addr, ops)]] + nxt
        else:
            succ[s] = nxt
    entry = {0: ()}
    work = [0]
    violations = {}
    deepest = 0
    rounds = 0
    while work:
        rounds += 1
        if rounds > 100000:
            raise RuntimeError("dataflow did not converge")
        s = work.pop()
        state = entry[s]
        b, e = blocks[s]
        for i in range(b, e):
            addr, mnem, ops = instrs[i]
            if mnem == "s_waitcnt":
                vm = vmcnt_of_waitcnt(ops)
                if vm is not None and vm < len(state):
                    state = state[len(state) - vm:]
                continue
            pending = frozenset().union(*state) if state else frozenset()
            hit = registers(ops) & pending
            if hit:
                violations[addr] = ("%s %s" % (mnem, ops), sorted(hit))
            if is_vmem(mnem):
                state = (state + (vmem_dest(mnem, ops),))[-MAX_VMCNT:]
                deepest = max(deepest, len(state))
        for t in succ[s]:
            new = state if t not in entry else merge(entry[t], state)
            if t not in entry or new != entry[t]:
                entry[t] = new
                work.append(t)
    if stats is not None:
        stats["vmem_ops"] = sum(1 for _, m, _ in instrs if is_vmem(m))
        stats["max_outstanding"] = deepest
    return [(a,) + violations[a] for a in sorted(violations)]


def check_library(lib: str, pattern: str = r"nvfp4_gem[mv]_kernel") -> dict:
    """{kernel: violations} for every function of `lib` whose name matches
    `pattern`; raises if no function matches."""
    funcs = parse(disassemble(lib))
    names = [f for f in funcs if re.search(pattern, f)]
    if not names:
        raise RuntimeError("no function matching %r in %s" % (pattern, lib))
    return {f: check_function(funcs[f]) for f in names}


def code_hash(lib: str, pattern: str = r"nvfp4_gemv_kernel") -> str:
    """sha256 prefix (16 hex digits) of the gfx950 code of every function of
    `lib` whose name matches `pattern`: names and instruction text in name
    order, without addresses.  It changes with the kernels' machine code and
    with nothing else (host code, other kernels)."""
    funcs = parse(disassemble(lib))
    names = sorted(f for f in funcs if re.search(pattern, f))
    if not names:
        raise RuntimeError("no function matching %r in %s" % (pattern, lib))
    h = hashlib.sha256()
    for f in names:
        h.update(f.encode() + b"\n")
        for _, mnem, ops in funcs[f]:
            h.update((mnem + " " + ops + "\n").encode())
    return h.hexdigest()[:16]
