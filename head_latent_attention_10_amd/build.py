"""Build the HIP library (libmla_hip.so) in-tree for gfx950 with hipcc.

Usage:  python -m head_latent_attention_10_amd.build   (always recompiles)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_hip.so")

SOURCES = ["mla_api.hip", "mla_small_kernels.hip", "mla_attend_simt.hip", "mla_attend_mfma.hip",
           "mla_attend_fp8.hip", "mla_proj_mfma.hip", "mla_cache_write.hip", "mla_dsa.hip",
           "mla_tpla.hip", "mla_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
    # never let the compiler form packed-fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the device code is compiled as above; the sanitizers instrument only
# the host code: argument checks, workspace layout, split arithmetic, launch
# sequencing).  Loaded with the sanitizer runtime preloaded (see
# asan_runtime()); used by the CPU test suite.
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libmla_hip_san.so")
SAN_FLAGS = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-shared-libasan"]


def asan_runtime() -> str | None:
    """The compiler's shared AddressSanitizer runtime (None if not installed)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_sanitized(verbose: bool = False) -> str:
    """Build SAN_LIB unless it is newer than every source and header."""
    os.makedirs(SAN_DIR, exist_ok=True)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    deps.append(os.path.join(ROOT, "include", "mla.h"))
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) > max(os.path.getmtime(d) for d in deps):
        return SAN_LIB

    def one(src: str) -> str:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *CFLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized) failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *SAN_FLAGS, *objs,
           "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build()
