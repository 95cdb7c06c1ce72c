"""Build libsparse_attn.so for gfx950 with hipcc (in-tree, no JIT cache).

Every translation unit is compiled for --offload-arch=gfx950 with packed
fp32 VALU instructions disabled, then linked into one shared library next to
this file.  ``python -m top_block_sparse_mean_amd.build`` does the same.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsparse_attn.so")
BUILD = os.path.join(PKG, "_build")
# The debugging build with contract checks (SA_CHECKED: gathers through the caller's
# device tables flag violations; sparse_attn_check_flags reads the flags).
CHECKED_OUT = os.path.join(PKG, "libsparse_attn_checked.so")
CHECKED_BUILD = os.path.join(PKG, "_build_checked")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Host-side address and undefined-behaviour checks for a test build (each flag applies to
# the host pass only; the GPU code is built as usual).  Load such a library with the
# compiler's address-sanitizer runtime preloaded and SPARSE_ATTN_LIB pointing at it.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def sanitizer_runtime() -> str:
    """The address-sanitizer runtime of the compiler hipcc drives (to preload)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = OUT, build_dir: str = BUILD,
          checked: bool = False) -> str:
    """Compile every source for gfx950 and link the library at `out`.  sanitize: host code
    with address and undefined-behaviour checks (a test build; see SANITIZE).  checked:
    kernels with contract checks (SA_CHECKED), by default at CHECKED_OUT."""
    if checked and out == OUT:
        out, build_dir = CHECKED_OUT, CHECKED_BUILD
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = (SANITIZE if sanitize else []) + (["-DSA_CHECKED"] if checked else [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] \
        if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, checked=True)
    sys.exit(0)
