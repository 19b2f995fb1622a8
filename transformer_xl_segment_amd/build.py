"""Build libtxl.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m transformer_xl_segment_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtxl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled for every kernel (the compiler would
# otherwise form them from float2-shaped code).
# Code object v5: loadable by the HIP runtime that ships with PyTorch, which the
# binding shares (torch's libamdhip64 is loaded first and satisfies libtxl's
# dependency on the same soname).
FLAGS = ["--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every source and link libtxl.so next to this file; return its path."""
    objs = []
    jobs = []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], "-c", src, "-o", obj]
        jobs.append((cmd, src))
        objs.append(obj)
    procs = [(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src)
             for cmd, src in jobs]
    failed = False
    for p, src in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"--- hipcc failed on {src}\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError("libtxl build failed")
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC",
                           *objs, "-o", tmp])
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
