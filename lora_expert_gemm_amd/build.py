"""Build the gfx950 HIP library ``_lib/libmoelora.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, into ``_build/`` and linked into one shared library
whose exported symbols are the C ABI of ``include/moelora.h``.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libmoelora.so")
SOURCES = ["api.hip", "align.hip", "expert_gemm.hip", "tiled_gemm.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _stale(src):
    """Whether src's object is older than src or any header of csrc/ or include/."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [
        os.path.join(d, f) for d in (CSRC, os.path.join(ROOT, "include"))
        for f in os.listdir(d) if f.endswith(".h")]
    return max(os.path.getmtime(p) for p in deps) > os.path.getmtime(obj)


def build(verbose=False, incremental=False):
    """Compile every source (incremental: only those whose object is stale) and link."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    with ThreadPoolExecutor(max(1, len(todo))) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
