"""Build ``liblr_attn.so`` in-tree for gfx950.

``plan.cpp``, ``rotate.cpp``, ``alloc.cpp`` and ``ffn_host.cpp`` (host-only
C++) are compiled with g++; ``ffn.hip`` joins the hipcc sources; ``kernels.hip``,
``project.hip`` and ``probe.hip`` with hipcc for gfx950; hipcc links them into
one shared library next to this file.  ``liblr_attn_check.so`` beside it is
the same library with ``kernels.hip``, ``ffn.hip`` and ``project.hip`` built
with ``LR_ATTN_CHECK=1`` (buffer accesses bounds-checked, a debugging aid).
"""
from __future__ import annotations

import json
import os
import re
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
# The host C++ under AddressSanitizer + UndefinedBehaviorSanitizer (gcc's
# runtimes, preloaded by the process that loads liblr_attn_san.so); the
# device code is the same.
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
SAN_LIB = os.path.join(HERE, "liblr_attn_san.so")
# The checked build (kernels with LR_ATTN_CHECK=1): a debugging aid.
CHECK_LIB = os.path.join(HERE, "liblr_attn_check.so")
HOST_SOURCES = ["plan.cpp", "rotate.cpp", "alloc.cpp", "ffn_host.cpp"]
HIP_SOURCES = ["ffn.hip", "kernels.hip", "project.hip", "probe.hip"]


# The compiler's per-kernel resource report (registers, spills, scratch,
# occupancy, LDS) for every HIP source; build() writes it to
# _build/kernel_resources.json.
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass-analysis=kernel-resource-usage\]")


def _run(cmd, resources=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if resources is not None:   # collect the resource remarks, keep them out of the log
        kernel = None
        for l in lines:
            m = _REMARK.search(l)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2)
            if key == "Function Name":
                kernel = val
                resources[kernel] = {}
            elif kernel is not None:
                resources[kernel][key] = val
        # the remarks and the source lines the compiler quotes under them
        lines = [l for l in lines if "kernel-resource-usage" not in l and not re.match(r"^\s*\d*\s*\|", l)]
    out = "\n".join(lines)
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
    res = {}
    outs = [
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "rotate.cpp"), "-o", rot_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "alloc.cpp"), "-o", alloc_o]),
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "ffn_host.cpp"), "-o", ffnh_o]),
        _run([HIPCC, *HIP_FLAGS, RESOURCE_FLAG, "-c", os.path.join(CSRC, "ffn.hip"), "-o", ffn_o], res),
        _run([HIPCC, *HIP_FLAGS, RESOURCE_FLAG, "-c", os.path.join(CSRC, "kernels.hip"), "-o", kern_o], res),
        _run([HIPCC, *HIP_FLAGS, RESOURCE_FLAG, "-c", os.path.join(CSRC, "project.hip"), "-o", proj_o], res),
        _run([HIPCC, *HIP_FLAGS, RESOURCE_FLAG, "-c", os.path.join(CSRC, "probe.hip"), "-o", probe_o], res),
    ]
    with open(os.path.join(BUILD, "kernel_resources.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, plan_o, rot_o, alloc_o, ffnh_o, ffn_o, kern_o,
                      proj_o, probe_o]))
    os.replace(tmp, LIB)
    outs.append(_build_checked([plan_o, rot_o, alloc_o, ffnh_o, probe_o]))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


def _build_checked(other_objs) -> str:
    """CHECK_LIB: kernels.hip, ffn.hip and project.hip rebuilt with
    LR_ATTN_CHECK=1 (every cache, workspace, weight, input and output access
    of their kernels tested against its buffer, lr_attn_check_count), linked
    with the host objects and the probe of the release build."""
    objs = []
    out = ""
    for src in ("kernels.hip", "ffn.hip", "project.hip"):
        o = os.path.join(BUILD, src.replace(".hip", "_check.o"))
        out += _run([HIPCC, *HIP_FLAGS, "-DLR_ATTN_CHECK=1", "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    tmp = CHECK_LIB + ".tmp"
    out += _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *other_objs, *objs])
    os.replace(tmp, CHECK_LIB)
    return out


def build_sanitized() -> str:
    """liblr_attn_san.so: the host sources rebuilt with SANITIZE_FLAGS, linked
    with the device objects of the last build() (built first if missing)."""
    hip_objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in HIP_SOURCES]
    if not all(os.path.exists(o) for o in hip_objs):
        build()
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    objs = []
    for s in HOST_SOURCES:
        o = os.path.join(san, s.replace(".cpp", ".o"))
        _run(["g++", *CXX_FLAGS, *SANITIZE_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs, *hip_objs])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose=True))
