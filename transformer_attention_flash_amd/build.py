"""Build libparallax.so in-tree for gfx950 with hipcc.

Usage:  python -m transformer_attention_flash_amd.build   (or build_library())
Each .hip translation unit is compiled in parallel into _build/, then linked
into transformer_attention_flash_amd/libparallax.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libparallax.so")
BUILD_INFO = os.path.join(PKG, "_build_info.json")  # git revision the library was built from
SOURCES = ["plx_api.hip", "plx_decode.hip", "plx_prefill.hip", "plx_backward.hip", "plx_projection.hip",
           "plx_diag.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the generated code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libparallax.so")


# Host-side sanitizers (the argument checks and launch policy run on the
# host); device code is built as usual.  Loading such a build needs the
# matching clang runtime preloaded (see sanitizer_runtime()).
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the HIP compiler's clang."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True) if os.path.isdir(root) else []:
        cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False, lib_path: str = LIB, host_sanitize: bool = False) -> str:
    """Compile every HIP source and link libparallax.so (always rebuilds).
    host_sanitize: build the host code with AddressSanitizer and
    UndefinedBehaviorSanitizer (for the CPU tests of the argument checks),
    into lib_path, which must then differ from the product library."""
    if host_sanitize and os.path.abspath(lib_path) == LIB:
        raise ValueError("a sanitizer build must not replace the product library")
    build_dir = os.path.join(BUILD, "host_sanitize") if host_sanitize else BUILD
    extra = HOST_SANITIZE_FLAGS if host_sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    # A sanitizer build links no runtime: the clang runtime, preloaded into the
    # process that loads the library, resolves the instrumentation.
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if host_sanitize:
        return lib_path
    _write_build_info()
    if verbose:
        print(f"built {LIB}")
    return LIB


def _write_build_info() -> None:
    """Record the git revision of the sources beside the library (the bench
    reports it; the GPU machines run a copy of the tree without .git)."""
    def git(*a):
        r = subprocess.run(["git", *a], cwd=ROOT, capture_output=True, text=True)
        return r.stdout.strip() if r.returncode == 0 else None

    sha = git("rev-parse", "HEAD")
    dirty = git("status", "--porcelain", "--untracked-files=no", "--", "transformer_attention_flash_amd", "include")
    info = {"git_sha": sha, "sources_modified_since_commit": bool(dirty) if dirty is not None else None,
            "built_at": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
