"""Builds libdblock.so for gfx950 with hipcc, in-tree.

    python -m block_wise_decoding_amd.build

Each HIP source is compiled to an object in parallel, then linked into
``block_wise_decoding_amd/libdblock.so`` (written to a temporary name and
renamed, so a half-written library is never loaded).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdblock.so")
SOURCES = ["api.hip", "commit.hip", "lmhead.hip", "lmhead_gemm.hip", "attend.hip", "cache.hip",
           "probe.hip"]
ARCH = "gfx950"

# hipcc flags: gfx950 only; packed fp32 instructions are disabled for every
# kernel (the compiler would otherwise fuse ordinary float pairs into them).
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: libdblock needs ROCm's hipcc to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)          # host-pass notice, harmless
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, s.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPFLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
