"""Build libm3.so (the HIP library behind include/m3.h) for gfx950, in-tree."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libm3.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else (shutil.which("hipcc") or "hipcc")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _clean(text: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so; drop that noise
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into libm3.so (always rebuilds). Each source is
    compiled to an object of its own, in parallel, then the objects are linked."""
    tag = "%d" % os.getpid()
    tmp = LIB + ".tmp" + tag
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    base = [hipcc()] + [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC]
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + "." + tag + ".o")
        cmd = base + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out = _clean(pr.communicate()[0])
        if pr.returncode != 0:
            failed.append("%s:\n%s" % (src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    try:
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + _clean(res.stdout))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
