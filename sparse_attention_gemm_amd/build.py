"""Build libdsa.so (gfx950) in-tree with hipcc.

    python -m sparse_attention_gemm_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.  Also builds libdsa_peaks.so, the measured-peak
microbenchmarks the benchmark reports next to the datasheet peaks.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def source_hash() -> str:
    """SHA-256 (first 16 hex digits) of every source the library is built from:
    the kernels, the host layer, their headers and include/dsa.h."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + [os.path.join(INCLUDE, "dsa.h")])
    for f in files:
        if os.path.isfile(f) and not f.endswith((".o", ".so")):
            h.update(os.path.relpath(f, ROOT).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile each source to an object in parallel, then link libdsa.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    stamp = source_hash()
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, f'-DDSA_SOURCE_HASH="{stamp}"', "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    build_peaks(verbose)
    return LIB


PEAKS_SRC = os.path.join(HERE, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libdsa_peaks.so")


def build_peaks(verbose: bool = False) -> str:
    """The measured-peak microbenchmarks the benchmark prices kernels against
    (a library of their own: they are not part of the path)."""
    tmp = PEAKS_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, PEAKS_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        sys.stderr.write(p.stdout.decode(errors="replace"))
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed for {src}")
    if verbose and lines:
        print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
