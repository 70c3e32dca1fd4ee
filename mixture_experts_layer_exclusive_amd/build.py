"""Builds the HIP library ``libmoe.so`` in-tree for gfx950 with hipcc.

Every source in ``csrc/`` is compiled to an object in parallel, then linked
into ``libmoe.so`` next to this file.  Run ``python -m
mixture_experts_layer_exclusive_amd.build`` or call :func:`build`.
"""
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and l.strip())
        if out:
            print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every csrc/*.hip and links libmoe.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizers for the CPU-only checks of the library's host layer
# (argument validation, workspace carving): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only, every flag behind
# -Xarch_host; the device code is compiled as usual (and never run by those
# checks).
SANITIZE_HOST_FLAGS = [
    "-O1", "-g", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a process loading the
    sanitized library must preload (its path, or "" if absent)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    for base in (llvm, "/opt/rocm/llvm/lib/clang"):
        if not os.path.isdir(base):
            continue
        for ver in sorted(os.listdir(base), reverse=True):
            so = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(so):
                return so
    return ""


def build_host_sanitized(out_dir: str) -> str:
    """Builds libmoe_sanitized.so into out_dir with SANITIZE_HOST_FLAGS; a
    process loads it with asan_runtime() preloaded and MOE_LIBRARY pointing
    at it.  Returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + SANITIZE_HOST_FLAGS

    def comp(src: str) -> str:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc(), *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(out_dir, "libmoe_sanitized.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
