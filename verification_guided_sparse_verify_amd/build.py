"""Build libvegas.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvegas.so")
PROBE_LIB = os.path.join(PKG, "libvegas_probe.so")
# Measurement build of the same sources with per-workgroup phase timestamps in
# the split kernel (VEGAS_PHASE_TRACE); loaded only by bench.py --phase-trace.
TRACE_LIB = os.path.join(PKG, "libvegas_trace.so")

SOURCES = ["attn.hip", "select.hip", "accept.hip", "api.cpp", "noalloc.cpp"]
PROBE_SOURCES = ["probe.hip"]      # measurement helper, its own library
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Build libvegas.so, libvegas_probe.so and libvegas_trace.so; returns the path of libvegas.so."""
    _build_lib(SOURCES, LIB, verbose)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose)
    _build_lib(SOURCES, TRACE_LIB, verbose, extra=["-DVEGAS_PHASE_TRACE"], subdir="trace")
    return LIB


def _build_lib(sources, lib, verbose: bool, extra=(), subdir: str = "") -> str:
    bdir = os.path.join(BUILD, subdir)
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if noise and (verbose or p.returncode):
            print("\n".join(noise), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs], check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
