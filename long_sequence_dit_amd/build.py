"""Build libattn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["attn_fwd_bf16.hip", "attn_fwd_f32.hip", "attn_fwd_fp8.hip", "lse_merge.hip", "ulysses_relayout.hip",
           "attn_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are disabled for every device compile.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so.  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


LIB_SAN = os.path.join(PKG, "libattn_san.so")
SAN_OBJDIR = os.path.join(PKG, "_build_san")


def build_sanitized(verbose: bool = False) -> str:
    """libattn_san.so: the host code of the C ABI (argument checks, chunk plan, workspace layout,
    shard driver) built with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    kernels' objects as built by build().  For the CPU sanitizer test, which loads it into a
    process whose AddressSanitizer runtime is preloaded.  The sanitizers apply to host code only:
    every -fsanitize flag is given to the host compilation alone (-Xarch_host)."""
    if not all(os.path.exists(os.path.join(OBJDIR, os.path.splitext(f)[0] + ".o")) for f in SOURCES):
        build(verbose)
    os.makedirs(SAN_OBJDIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    api_obj = os.path.join(SAN_OBJDIR, "attn_api.o")
    cmd = [HIPCC] + COMMON + san + ["-x", "hip", "-c", os.path.join(CSRC, "attn_api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized attn_api.cpp:\n%s\n%s" % (" ".join(cmd), res.stderr))
    objs = [api_obj] + [os.path.join(OBJDIR, os.path.splitext(f)[0] + ".o") for f in SOURCES if f != "attn_api.cpp"]
    tmp = LIB_SAN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB_SAN)
    if verbose:
        print("built", LIB_SAN)
    return LIB_SAN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
