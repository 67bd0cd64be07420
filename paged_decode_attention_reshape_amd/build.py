"""Builds libkv4.so (the C-ABI HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkv4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: every kernel uses scalar fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# The attention kernels use +-inf but never NaN: let max/min skip NaN quieting.
# (The write path stays on default IEEE semantics: its results are compared
# bit for bit.)
# Matrix-core accumulators stay in ordinary VGPRs (the softmax rescale and
# the epilogue touch them with VALU ops; AGPR copies would cost both).
PER_FILE = {
    "kv4_attn_mfma.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kv4_attn_prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kv4_attn_valu.hip": ["-fno-honor-nans"],
}


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source under csrc/ and link libkv4.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Debug build: the same sources with -DKV4_DEBUG, whose kernels also record
# every input they clamp or skip (kv4_debug_flags in include/kv4.h), linked
# as libkv4_debug.so next to the release library. Load it in place of the
# release library by setting KV4_LIBRARY to its path before the binding's
# first call.
DEBUG_LIB = os.path.join(PKG, "libkv4_debug.so")
DEBUG_BUILD = os.path.join(BUILD, "debug")


def build_debug_library(verbose: bool = False) -> str:
    os.makedirs(DEBUG_BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, DEBUG_BUILD, ("-DKV4_DEBUG",)), SOURCES))
    tmp = DEBUG_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"debug link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DEBUG_LIB)
    return DEBUG_LIB


# Host-side sanitizers for the C ABI's validation and planner (kv4_api.cpp):
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
# GPU code objects are built as usual), linked with the other objects of the
# regular build. Loading it needs the clang ASan runtime preloaded.
SAN_LIB = os.path.join(BUILD, "asan", "libkv4_asan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc (None if absent)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized_library(verbose: bool = False) -> str:
    """libkv4 with kv4_api.cpp built under ASan + UBSan (host code)."""
    objs = [os.path.join(BUILD, os.path.splitext(f)[0] + ".o") for f in SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build_library(verbose)
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    api_obj = os.path.join(os.path.dirname(SAN_LIB), "kv4_api.o")
    cmd = [HIPCC, "-x", "hip", *COMMON, "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, "kv4_api.cpp"),
           "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized kv4_api.cpp:\n{r.stdout}\n{r.stderr}")
    others = [o for o in objs if not o.endswith("kv4_api.o")]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libasan", "-o", SAN_LIB,
           api_obj, *others]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the sanitized library failed:\n{r.stdout}\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
