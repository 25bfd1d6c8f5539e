"""Build libpkv.so, libpkv_checked.so and libpkv_calib.so (HIP, gfx950)
in-tree with hipcc.

Every source under csrc/ is compiled to an object in parallel and linked
into ``paged_kv_cache_prepare_amd/libpkv.so``.  The checked build
(``libpkv_checked.so``) links the same kernels with api.hip compiled again
under ``PKV_DEBUG_CHECKS`` and the validation kernels of checks.hip.  The
benchmark's measurement kernels (csrc/calib/calib.hip, include/pkv_calib.h)
are a library of their own, ``libpkv_calib.so``.
Packed-fp32 instructions are switched off for all device code
(``-packed-fp32-ops``).  ``FILE_FLAGS`` adds per-file options.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpkv.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libpkv_checked.so")
CALIB_LIB_PATH = os.path.join(HERE, "libpkv_calib.so")
KERNEL_SOURCES = ["prepare.hip", "kv_write.hip", "block_ops.hip", "attention.hip"]
SOURCES = ["api.hip", *KERNEL_SOURCES]
# Per-file flags.  The attention kernels never feed a NaN into a max or a sum
# (masked scores are selected away first), so max operations need no NaN
# canonicalisation.
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libpkv needs the ROCm toolchain")


def compile_flags(extra=()) -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra]


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile and link libpkv.so and libpkv_checked.so.  Always rebuilds.
    Returns the path of libpkv.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def one(job):
        src, name, flags = job
        obj = os.path.join(BUILD_DIR, name)
        cmd = [cc, *compile_flags([*FILE_FLAGS.get(src, []), *flags, *extra_flags]), "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    jobs = [(src, src.rsplit(".", 1)[0] + ".o", []) for src in SOURCES]
    jobs += [("api.hip", "api_checked.o", ["-DPKV_DEBUG_CHECKS"]), ("checks.hip", "checks.o", []),
             (os.path.join("calib", "calib.hip"), "calib.o", [])]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = dict(zip((j[1] for j in jobs), ex.map(one, jobs)))
    kernels = [objs[src.rsplit(".", 1)[0] + ".o"] for src in KERNEL_SOURCES]
    for path, own in ((LIB_PATH, [objs["api.o"]]),
                      (CHECKED_LIB_PATH, [objs["api_checked.o"], objs["checks.o"]]),
                      (CALIB_LIB_PATH, [objs["calib.o"]])):
        if path == CALIB_LIB_PATH:
            kernels_of = []
        else:
            kernels_of = kernels
        tmp = path + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *own, *kernels_of, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
