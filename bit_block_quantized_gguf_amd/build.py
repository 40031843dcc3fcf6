"""Build libq4k.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only.  Packed FP32 VALU
instructions are disabled in device code (-packed-fp32-ops); the host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libq4k.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # code object v5: loadable by the ROCm 7.0 runtime bundled with torch as
    # well as by the system 7.2 runtime (the library binds to whichever
    # libamdhip64.so.7 is already in the process)
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libq4k.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), max(1, (os.cpu_count() or 2)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-mcode-object-version=5", "-shared", "-fPIC",
           "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
