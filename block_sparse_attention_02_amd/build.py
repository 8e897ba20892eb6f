"""Builds libh3attn.so (all HIP sources in csrc/) for gfx950 with hipcc, in-tree.

Usage: python -m block_sparse_attention_02_amd.build [--sanitize]

--sanitize builds _build_san/libh3attn_san.so instead: the same sources with the host
code (argument checks, workspace layout, the partition planner) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer; device code is built as usual. Load it
with H3ATTN_LIB pointing at it and the ASan runtime preloaded (see san_runtime()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libh3attn.so")
ARCH = os.environ.get("H3ATTN_ARCH", "gfx950")

# Packed float32 VALU instructions are disabled for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-Wno-unused-variable"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libh3attn)")


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# The router's pooled scores are defined as separately rounded products and sums,
# so no multiply-add may be contracted anywhere in that file.
PER_FILE = {"router.hip": ["-ffp-contract=off"]}


# host-only sanitizer flags: each -fsanitize= applies to the host pass alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-g"]
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libh3attn_san.so")


def _compile(hipcc: str, src: str, build_dir: str = BUILD, san: bool = False) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    extra = PER_FILE.get(os.path.basename(src), []) + (SAN_FLAGS if san else [])
    cmd = [hipcc, *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compiles every csrc/*.hip and links libh3attn.so next to this file."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """Builds the host-sanitized library (see the module docstring); returns its path."""
    hipcc = _hipcc()
    os.makedirs(SAN_BUILD, exist_ok=True)
    srcs = _sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, SAN_BUILD, True), srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fsanitize=address",
           "-fsanitize=undefined", "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def san_runtime() -> str:
    """Path of the ASan runtime the sanitized library links against (to preload into an
    uninstrumented interpreter)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
