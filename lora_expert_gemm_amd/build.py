"""Build the gfx950 HIP library ``_lib/libmoelora.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, into ``_build/`` and linked into one shared library
whose exported symbols are the C ABI of ``include/moelora.h``.
"""
import json
import os
import re
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


# Sources whose GEMM kernels wait on counts of their own vector-memory loads
# (s_waitcnt vmcnt with a fixed immediate): a scratch spill reload is a
# vector load too, so every kernel of these must use no scratch memory.
COUNTED_WAITS = ("expert_gemm.hip", "tiled_gemm.hip")
# The device assembly of the streaming GEMMs is kept for the CPU test that
# checks the compiled weight-ring loops against their wait counts.
ASM_SOURCES = ("expert_gemm.hip",)
_NOISE = "is not a recognized feature for this target"  # host pass, packed-fp32 flag
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|"
                     r"SGPRs Spill|VGPRs|AGPRs|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]): (\S+)")


def _resources(stderr):
    """Per-kernel resource usage from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.isdigit() else val
    return out


def _run(cmd, src):
    p = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in p.stderr.splitlines()
                    if _NOISE not in l and "kernel-resource-usage" not in l
                    and not re.match(r"^\s*(\d+\s*)?\|", l) and not l.startswith("  ")
                    and l.strip() != "")
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return p.stderr


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src in COUNTED_WAITS else []
    stderr = _run([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], src)
    if src in COUNTED_WAITS:
        res = _resources(stderr)
        with open(os.path.join(BUILD, src + ".resources.json"), "w") as f:
            json.dump(res, f, indent=0, sort_keys=True)
        bad = [k for k, v in res.items()
               if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0) or v.get("SGPRs Spill", 0)]
        if bad:
            raise RuntimeError(f"{src}: kernels with counted waits use scratch or spill: {bad}")
    return obj


def _assemble(src):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + "-gfx950.s")
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out], src)
    return out


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
    with ThreadPoolExecutor(max(1, len(todo) + len(ASM_SOURCES))) as ex:
        jobs = [ex.submit(_compile, s) for s in todo]
        jobs += [ex.submit(_assemble, s) for s in ASM_SOURCES if s in todo]
        for j in jobs:
            j.result()
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
