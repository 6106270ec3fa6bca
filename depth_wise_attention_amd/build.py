"""Build libattnres.so for gfx950 with hipcc (in-tree, next to this file).

Every .hip / .cpp source under csrc/ is compiled to an object in _build/ and
linked into depth_wise_attention_amd/libattnres.so.  Packed FP32 instructions
are disabled on the device pass (-packed-fp32-ops).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattnres.so")
ARCH = os.environ.get("ATTNRES_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link the shared library; returns its path.

    `defines` (e.g. ["-DATTNRES_P1_PREFETCH=0"]) override the kernels'
    compile-time tuning knobs; such builds go to their own object directory."""
    bdir = BUILD if out == LIB else os.path.join(BUILD, os.path.basename(out) + ".d")
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        out_ = _run([cc, *COMMON, *defines, *lang, "-c", src, "-o", obj])
        if verbose and out_.strip():
            print(out_)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(CSRC, "probe", "stream_pattern.hip")
PROBE_LIB = os.path.join(PKG, "libattnres_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Build the streaming-pattern probe (bench.py --ceilings) into its own
    library; it is not part of libattnres.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    obj = os.path.join(BUILD, "stream_pattern.hip.o")
    out_ = _run([cc, *COMMON, "-c", PROBE_SRC, "-o", obj])
    if verbose and out_.strip():
        print(out_)
    tmp = PROBE_LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj])
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
    print(build_probe(verbose="-v" in sys.argv))
