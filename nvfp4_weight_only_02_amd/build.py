"""Build the HIP libraries (gfx950) in-tree with hipcc.

``python -m nvfp4_weight_only_02_amd.build`` compiles libnvfp4.so (the decode
projection, C ABI in include/nvfp4.h) and libnvfp4_probes.so (measurement
aids beside it, include/nvfp4_probes.h).  The flags keep hipcc from emitting
packed-fp32 VALU instructions (``-packed-fp32-ops``) for every kernel.  A
build of libnvfp4.so is refused if a GEMV or GEMM kernel spills or uses
scratch, or if its disassembly shows a register of an in-flight load touched
before the wait that covers the load (asmcheck.py).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnvfp4.so")
PROBES_LIB = os.path.join(PKG, "libnvfp4_probes.so")
# (library, its sources)
TARGETS = [(LIB, [os.path.join(PKG, "csrc", "nvfp4.hip")]),
           (PROBES_LIB, [os.path.join(PKG, "csrc", "probes.hip")])]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def check_resources(remarks: str) -> None:
    """Refuse a build in which a GEMV or GEMM kernel spills registers or uses scratch.

    These kernels issue their vector-memory loads as inline assembly and
    wait for them with explicit vmcnt counts; the compiler does not know such
    a load is still in flight, so a spill (or any other copy) of its
    destination registers before the wait would read them too early."""
    kernel = None
    bad = []
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        if kernel is None or ("gemv_kernel" not in kernel and "gemm_kernel" not in kernel):
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) != 0:
            bad.append("%s: %s = %s" % (kernel, m.group(1), m.group(2)))
    if bad:
        raise RuntimeError("GEMV/GEMM kernels must not spill or use scratch:\n  " + "\n  ".join(bad))


def check_inflight(lib: str) -> None:
    """Refuse a build in which any GEMV or GEMM kernel names a register that a
    vector-memory load may still be writing (asmcheck.py: a dataflow over the
    disassembly of the gfx950 code just built).  The kernels' hand-counted
    vmcnt waits are only right if the compiler keeps every such register
    untouched until the wait that covers its load."""
    from . import asmcheck   # noqa: PLC0415 (build.py also runs as a script)
    found = {k: v for k, v in asmcheck.check_library(lib).items() if v}
    if found:
        lines = []
        for kernel, hits in sorted(found.items()):
            for addr, text, regs in hits[:3]:
                lines.append("%s +%#x: %s (in flight: %s)" % (kernel, addr, text, regs[:4]))
        raise RuntimeError("registers of in-flight loads are touched before their wait:\n  " + "\n  ".join(lines))


def build_one(lib: str, sources: list, verbose: bool = False) -> str:
    """Compile one library (always) and return its path."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-Rpass-analysis=kernel-resource-usage"] + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [line for line in res.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in line]
    # Drop the resource remarks and the source lines clang quotes under them.
    kept, after_remark = [], False
    for line in lines:
        if "remark:" in line:
            after_remark = True
            continue
        if after_remark and re.match(r"^\s*(\d+\s*)?\|", line):
            continue
        after_remark = False
        kept.append(line)
    out = "\n".join(kept)
    try:
        check_resources("\n".join(lines))
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + out)
        if lib == LIB:
            check_inflight(tmp)
    except RuntimeError:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every library (always); returns the path of libnvfp4.so."""
    for lib, sources in TARGETS:
        build_one(lib, sources, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
