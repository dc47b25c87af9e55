"""Build libpa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: ``python -m paged_kv_cache_page_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``paged_kv_cache_page_amd/_build/``; the library to
``paged_kv_cache_page_amd/libpa.so``.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

# Per-file extra flags. The RoPE/cache-write unit rounds every product and sum
# separately, so contraction into fused multiply-adds is off there; it also
# compiles the plan (pa_plan.h), which the plan kernel's unit then compiles
# with the same flag.
EXTRA = {"pa_rope_cache.hip": ["-ffp-contract=off"], "pa_plan.hip": ["-ffp-contract=off"],
         "pa_sample.hip": ["-ffp-contract=off"]}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    # packed-FP32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpa")
    return path


# Host-only C++ sources (the block manager) are compiled by the host compiler.
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [shutil.which("g++") or "g++", *HOST_FLAGS, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    return obj, warn


def build(verbose=False):
    """Compile every HIP (and host C++) source and link libpa.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                     if f.endswith(".hip") or f.endswith(".cpp"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        results = list(ex.map(_compile, sources))
    for obj, warn in results:
        if warn and verbose:
            print(f"[{os.path.basename(obj)}] {warn}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
           *[o for o, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
