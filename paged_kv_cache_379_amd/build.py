"""Build libpkv.so in place: hipcc for gfx950, one object per source, in parallel.

Run ``python -m paged_kv_cache_379_amd.build`` (or call ``build()``); the
library lands next to this file and the objects under ``_build/``.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed fp32 instructions off (the host pass warns
# that it does not know the feature; that warning is harmless).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA accumulators in ordinary VGPRs (no copies to and from AGPRs
          # around the vector code that rescales them)
          "-mllvm", "-amdgpu-mfma-vgpr-form"]

SOURCES = [
    "errors.cpp",
    "allocator.cpp",
    "decode.hip",
    "decode_f32.hip",
    "decode_f16.hip",
    "decode_bf16.hip",
    "decode_i8.hip",
    "decode_fp8.hip",
    "cache_write.hip",
]


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link libpkv.so (always rebuilds)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libpkv.so failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
