"""Build libspax.so in-tree with hipcc for gfx950.

    python activation_sparse_tiered_amd/build.py       # or __graft_entry__.build()

Every source under csrc/ is compiled as HIP for gfx950 and linked into
activation_sparse_tiered_amd/libspax.so.  Objects go to _build/ at the repository root.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspax.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-mcode-object-version=5",
    "-Wno-unused-function", "-Wno-unused-variable",
    # no packed fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["host.cpp", "api.cpp", "pack.hip", "tiers.hip", "gemv.hip", "decode.hip", "batch.hip",
           "pinned.cpp", "probe.hip", "budgets.cpp"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = (r.stderr or "").strip()
    if warn:
        # hipcc's host pass does not know the packed-fp32 feature flag; anything else is shown
        lines = [ln for ln in warn.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    write_buildinfo(LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def write_buildinfo(lib: str) -> None:
    """Record how the library `lib` was built (flags without include paths, compiler banner) in
    `lib`.buildinfo, so that measurements can be tied to the build without running the compiler
    later.  The path follows the library actually written, so a build elsewhere leaves the
    package's record alone."""
    r = subprocess.run([hipcc(), "--version"], capture_output=True, text=True)
    banner = " ".join(r.stdout.split())
    flags = " ".join(f for f in FLAGS if not f.startswith("-I"))
    with open(lib + ".buildinfo", "w") as fh:
        fh.write(f"flags: {flags}\ncompiler: {banner}\n")


if __name__ == "__main__":
    build(verbose=True)
