"""Build libyoco.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m yoco_shared_kv_gather_amd.build`` (or ``build()`` from
Python).  Every source compiles to an object in ``_build/`` in parallel, then
one link step writes ``libyoco.so`` next to this file.  The standalone check
programs under ``tests/`` (hardware facts the kernels rely on) build alongside.  Packed fp32 VALU
instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libyoco.so")

SOURCES = ["abi.hip", "gather_last.hip", "kv_append.hip", "cross_attn.hip", "cross_attn_f32.hip", "cross_attn_bf16.hip",
           "cross_attn_fp8.hip", "cross_attn_mfma_bf16.hip", "cross_attn_mfma_fp8.hip", "retention.hip", "validate.hip"]

# Standalone GPU check programs the tests run (source, binary), built with the library.
CHECKS = [(os.path.join(ROOT, "tests", "e4m3_encoder_check.hip"), os.path.join(ROOT, "tests", "e4m3_encoder_check"))]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libyoco.so")
    return path


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libyoco.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src, exe in CHECKS:
        cmds.append([cc, *COMMON_FLAGS, src, "-o", exe])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        for out in pool.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libyoco_asan.so")
# AddressSanitizer on the host half only: each -fsanitize applies to the host
# compilation (device code is built exactly as in the library).
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The AddressSanitizer runtime that must be preloaded into the process
    that loads the instrumented library."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL, text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("AddressSanitizer runtime not found")
    return found[-1]


def build_asan(jobs: int = 8) -> str:
    """A copy of the library whose host code (argument checks, launch set-up,
    validation) is built with AddressSanitizer, for the CPU tests of the C
    ABI.  Rebuilt only when a source changed."""
    import hashlib
    os.makedirs(ASAN_DIR, exist_ok=True)
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)) + ["../../include/yoco.h"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    h.update(" ".join(COMMON_FLAGS + ASAN_FLAGS).encode())
    stamp = os.path.join(ASAN_DIR, "sources.sha256")
    digest = h.hexdigest()
    if os.path.exists(ASAN_LIB_PATH) and os.path.exists(stamp) and open(stamp).read() == digest:
        return ASAN_LIB_PATH
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, *ASAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(_run, cmds))
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", *objs, "-o",
          ASAN_LIB_PATH])
    with open(stamp, "w") as f:
        f.write(digest)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan())
    else:
        print(build(verbose="-v" in sys.argv))
