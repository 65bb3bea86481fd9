"""Build libstem.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m block_sparse_attention_oam_amd.build   (or call build()).
Each .hip file compiles to an object in _build/ in parallel, then they link into
block_sparse_attention_oam_amd/libstem.so.

python -m block_sparse_attention_oam_amd.build --host-sanitizers (or build_host_sanitized()) builds the
same library with its host code (validation, planning, budgets, launch set-up) under AddressSanitizer and
UndefinedBehaviorSanitizer into _build/host_san/libstem.so; device code is compiled as usual.  Load it
with STEM_LIB pointing there and the runtime that asan_runtime() names preloaded.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libstem.so")

SOURCES = ["stem_api.hip", "pool_score.hip", "tpd_topk.hip", "score_topk.hip", "naive_score.hip", "bsa_fwd.hip", "bsa_bf16.hip", "bsa_fp8.hip"]

# Packed-fp32 VALU ops are disabled for all device code; the host pass warns that it does not know the
# feature, which is harmless.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Host-side sanitizer flags: every -fsanitize applies to the host pass only (-Xarch_host).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_DIR = os.path.join(BUILD, "host_san")


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (it carries the UBSan handlers too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src: str, objdir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


def build_host_sanitized(verbose: bool = True, jobs: int = 0) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, SAN_DIR, tuple(SAN_FLAGS)), SOURCES))
    out = os.path.join(SAN_DIR, "libstem.so")
    rt = os.path.dirname(asan_runtime())
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
           "-shared-libasan", "-Wl,-rpath," + rt, "-o", out + ".tmp", *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv[1:]:
        build_host_sanitized()
    else:
        build()
