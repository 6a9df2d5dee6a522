"""Build libkda.so (the C-ABI library of include/kda.h) with hipcc for gfx950.

Every .hip file under csrc/ is compiled to an object in parallel and linked
into linear_attention_05_amd/libkda.so, in-tree. Run as a script or call
build(). Packed fp32 VALU instructions are disabled for all device code."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
OBJDIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda.so)")


def common_flags():
    # -packed-fp32-ops: no packed fp32 instructions in generated code.
    # -amdgpu-mfma-vgpr-form: matrix-core results in ordinary VGPRs, so the
    # scan's state takes part in vector arithmetic without register copies.
    return ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *common_flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr, flush=True)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(PKG, "_build", "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libkda_hostsan.so")


def build_host_sanitized(verbose: bool = False, jobs: int = 8) -> str:
    """The library with its host code (argument validation, workspace sizing,
    launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer,
    for CPU tests of the C ABI; device code as in build(). Load it with the
    matching sanitizer runtime preloaded. Rebuilt only when a source or header
    is newer than it."""
    cc = hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()
    deps = srcs + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)] + [os.path.abspath(__file__)]
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > max(os.path.getmtime(d) for d in deps):
        return SAN_LIB
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *common_flags(), "-g", *san, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *san,
           "-o", SAN_LIB, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (with UBSan)."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if not out or not os.path.exists(out):
        raise RuntimeError("shared AddressSanitizer runtime not found")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
