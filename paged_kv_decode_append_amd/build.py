"""Compile the HIP sources under csrc/ into libpkv.so for gfx950 (in-tree).

Usage: python paged_kv_decode_append_amd/build.py [-v] [--sanitize]   (or __graft_entry__.build()).
Run it by path: importing the package loads libpkv.so, which may not exist yet.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
BUILD_DIR = os.path.join(ROOT, "_build", "pkv")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


HOST_CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]

# Host code with AddressSanitizer + UndefinedBehaviorSanitizer (build(sanitize=True)):
# every host part -- the block manager / scheduler and the host side of the
# .hip sources (entry points, argument checks, plans, pkv_validate_step) --
# is built by clang, so that one sanitizer runtime serves the process (load
# the library with SAN_RUNTIME preloaded).  Device code is built as usual:
# on hipcc lines each sanitizer flag goes to the host pass only.
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libpkv.so")
SAN_CXX = os.environ.get("SAN_CXX", "/opt/rocm/llvm/bin/clang++")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def san_runtime() -> str | None:
    """clang's shared AddressSanitizer runtime (it carries the UBSan handlers)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):  # host-only sources (the block manager / scheduler)
        if sanitize:
            cmd = [SAN_CXX, *HOST_FLAGS, *SAN_FLAGS, "-c", src, "-o", obj]
        else:
            cmd = [HOST_CXX, *HOST_FLAGS, "-c", src, "-o", obj]
    else:
        host_san = [x for f in SAN_FLAGS for x in ("-Xarch_host", f)] if sanitize else []
        cmd = [HIPCC, *COMMON_FLAGS, *host_san, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libpkv.so in-tree; with sanitize, the host-sanitized build at
    SAN_LIB instead (the in-tree library is left alone)."""
    os.makedirs(SAN_DIR if sanitize else BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), sources))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    san_link = ["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san_link, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
