"""Build ``liblr_attn.so`` in-tree for gfx950.

``plan.cpp``, ``rotate.cpp``, ``alloc.cpp`` and ``ffn_host.cpp`` (host-only
C++) are compiled with g++; ``ffn.hip`` joins the hipcc sources; ``kernels.hip``,
``project.hip`` and ``probe.hip`` with hipcc for gfx950; hipcc links them into
one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblr_attn.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are switched off: hipcc forms them from ordinary
# float code, and the kernels do not need them.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    plan_o = os.path.join(BUILD, "plan.o")
    rot_o = os.path.join(BUILD, "rotate.o")
    alloc_o = os.path.join(BUILD, "alloc.o")
    ffnh_o = os.path.join(BUILD, "ffn_host.o")
    ffn_o = os.path.join(BUILD, "ffn.o")
    kern_o = os.path.join(BUILD, "kernels.o")
    proj_o = os.path.join(BUILD, "project.o")
    probe_o = os.path.join(BUILD, "probe.o")
    outs = [
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "rotate.cpp"), "-o", rot_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "alloc.cpp"), "-o", alloc_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "ffn_host.cpp"), "-o", ffnh_o]),
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "ffn.hip"), "-o", ffn_o]),
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "kernels.hip"), "-o", kern_o]),
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "project.hip"), "-o", proj_o]),
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "probe.hip"), "-o", probe_o]),
    ]
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, plan_o, rot_o, alloc_o, ffnh_o, ffn_o, kern_o,
                      proj_o, probe_o]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
