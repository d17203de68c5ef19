"""Build libkda.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m chunked_kda_prefill_amd.build  (or __graft_entry__.build()).
"""

from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the recurrence rescales and converts
    # its state every chunk, which costs AGPR<->VGPR moves otherwise
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_hash() -> str:
    """Short sha256 over every file the library is built from (sources,
    headers, the public header and this file's flags).  Counter readings
    taken for one build are only valid while this value is unchanged."""
    files = sorted(glob.glob(os.path.join(CSRC, "*"))) + [
        os.path.join(ROOT, "include", "kda.h"), os.path.abspath(__file__)]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_files(unit: str):
    """The translation unit csrc/<unit> and every csrc header it includes,
    directly or not."""
    import re
    todo, seen = [unit], []
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.append(f)
        with open(os.path.join(CSRC, f)) as fh:
            todo += re.findall(r'^#include "([^"]+)"', fh.read(), re.M)
    return sorted(seen)


def kernel_hash(unit: str) -> str:
    """Short sha256 over one kernel's sources (kernel_files) and the compile
    flags: counter readings of that kernel stay valid while it is unchanged,
    whatever else in the library changes."""
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for f in kernel_files(unit):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the kernels whose counters the bench reports, by translation unit
KERNEL_UNITS = {"kda_intra": "kda_intra.hip", "kda_recurrence": "kda_recurrence.hip"}


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if errs and verbose:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
