"""Build liblconv.so (HIP for gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection disabled (the compiler
otherwise forms v_pk_*_f32 from ordinary float code).  Works without a GPU: hipcc
cross-compiles the device code for gfx950.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblconv.so")

ARCH = "gfx950"
HIP_SOURCES = ["fused1d_conv.hip", "fused1d_adj.hip", "fused1d_part.hip", "fused1d_sparse.hip", "fused1d_save.hip",
               "fused1d.hip", "bwd1d.hip", "multipass.hip", "fftconv2d.hip", "fftconv3d.hip",
               "stage.hip", "ssm.hip", "noalloc.hip", "colmx.hip", "butterfly.hip", "fused1d_lbf.hip"]
CPP_SOURCES = ["plan.cpp", "lconv_api.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def _deps(src: str) -> set:
    """src and every project header it includes, directly or through other headers."""
    import re
    seen, todo = set(), [src]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(f):
            continue
        seen.add(f)
        for name in re.findall(r'^\s*#\s*include\s+"([^"]+)"', open(f).read(), flags=re.M):
            for d in (CSRC, INCLUDE):
                cand = os.path.join(d, name)
                if os.path.exists(cand):
                    todo.append(cand)
                    break
    return seen


def _stale(obj: str, src: str) -> bool:
    """True when obj is missing or older than its source or a header it includes."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in _deps(src))


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    """Compile every source (only the stale ones with incremental=True) and link liblconv.so;
    returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        src = os.path.join(CSRC, s)
        if not os.path.exists(src):
            continue
        obj = os.path.join(BUILD, s + ".o")
        if not incremental or _stale(obj, src):
            cmds.append([hipcc, *COMMON, *DEVICE, "-c", src, "-o", obj])
        objs.append(obj)
    for s in CPP_SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s + ".o")
        if not incremental or _stale(obj, src):
            cmds.append([hipcc, *COMMON, "-c", src, "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
