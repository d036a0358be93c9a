"""Compile the HIP sources under ``csrc/`` into ``libpsq.so`` for gfx950.

Each translation unit is compiled in parallel with hipcc, then linked into
one shared library next to this file (in-tree, so it travels with the
source tree).  The result is written to a temporary name and renamed, so a
reader never sees a half-written library.

The same sources are also built with ``PSQ_JITTER`` into
``libpsq_jitter.so``: the race-test build, whose workgroups sleep a random
time at each step of a cross-workgroup protocol.  Only the tests load it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpsq.so")
JITTER_LIB = os.path.join(HERE, "libpsq_jitter.so")
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of every code object; the host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the psq library needs ROCm's hipcc")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Build ``libpsq.so`` and the race-test build ``libpsq_jitter.so``."""
    _build_one(LIB, [], verbose)
    _build_one(JITTER_LIB, ["-DPSQ_JITTER"], verbose)
    return LIB


def _build_one(lib_path: str, defines: list, verbose: bool) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="psq_build_") as tmp:
        procs = []
        objs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIP_FLAGS, *defines, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = "\n".join(l for l in out.splitlines()
                             if "packed-fp32-ops" not in l)
            if pr.returncode != 0:
                failed.append(f"{src}:\n{text}")
            elif verbose and text.strip():
                print(text, flush=True)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        tmp_lib = lib_path + ".tmp"
        cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib, *objs]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
