"""Build ``libmoe_gfx950.so`` from ``csrc/*.hip`` with hipcc for gfx950.

Each source compiles to its own object (in parallel) under ``_build/`` at the
repository root; the objects link into the in-tree shared library next to this
file.  Run ``python -m expert_gemms_amd.build`` or call ``build()``.

``build(sanitize=True)`` makes a second library under ``_build/host_asan/``
whose host code is instrumented by AddressSanitizer and UndefinedBehavior-
Sanitizer (device code unchanged), for the CPU tests of the host-side logic;
it is rebuilt only when a source or a flag changes.  It needs the ASan
runtime preloaded (``asan_runtime()``).
"""

import concurrent.futures
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_gfx950.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", SRC,
    # packed FP32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# host-side sanitizers (each -fsanitize= applies to the host compilation only)
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
ASAN_BUILD_DIR = os.path.join(BUILD_DIR, "host_asan")
ASAN_LIB = os.path.join(ASAN_BUILD_DIR, "libmoe_gfx950_host_asan.so")


def asan_runtime():
    """Path of the compiler's ASan runtime (to preload), or None."""
    pat = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "lib", "clang", "*", "lib", "linux",
                       "libclang_rt.asan-x86_64.so")
    hits = sorted(glob.glob(pat)) or sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


# the GEMM kernels' register report (VGPRs, spills, scratch per kernel), written
# by the library build for tests/test_gemm_registers.py
GEMM_USAGE = os.path.join(BUILD_DIR, "gemm.resource-usage.txt")
GEMM_USAGE_SOURCES = ("gemm.hip", "common.h", "launch.h", "l2input.h")


def gemm_sources_sha256():
    h = hashlib.sha256(" ".join([HIPCC, *FLAGS]).encode())
    for f in GEMM_USAGE_SOURCES:
        with open(os.path.join(SRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


def _compile(src, build_dir=BUILD_DIR, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    usage = not extra and os.path.basename(src) == "gemm.hip"
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj] + (["-Rpass-analysis=kernel-resource-usage"] if usage else [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if usage:
        with open(GEMM_USAGE, "w") as fh:
            fh.write(f"sources sha256 {gemm_sources_sha256()}\n")
            fh.write("\n".join(l for l in r.stderr.splitlines() if "remark" in l) + "\n")
    return obj


def _sources():
    return sorted(os.path.join(SRC, f) for f in os.listdir(SRC) if f.endswith(".hip"))


def _stamp(extra):
    h = hashlib.sha256(" ".join([HIPCC, *FLAGS, *extra]).encode())
    for f in sorted(os.listdir(SRC)) + sorted(os.listdir(INCLUDE)):
        d = SRC if os.path.exists(os.path.join(SRC, f)) else INCLUDE
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


def build(verbose=False, sanitize=False):
    build_dir, lib, extra = (ASAN_BUILD_DIR, ASAN_LIB, SANITIZE_FLAGS) if sanitize else (BUILD_DIR, LIB, [])
    os.makedirs(build_dir, exist_ok=True)
    stamp_file = os.path.join(build_dir, "sources.sha256")
    if sanitize:
        stamp = _stamp(extra)
        if os.path.exists(lib) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
            return lib
    srcs = _sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if sanitize:
        with open(stamp_file, "w") as fh:
            fh.write(stamp)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
