"""Build libhisa.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m long_context_indexer_block_amd.build [--jobs N] [--sanitize]

--sanitize builds a second copy, _build/sanitize/libhisa_sanitize.so, whose
host code (argument validation, error text, workspace carving, launch set-up)
runs under AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is
compiled as usual. It is a test build: load it with the clang ASan runtime
preloaded (sanitizer_runtime()) and HISA_LIBRARY naming it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhisa.so")
ARCH = "gfx950"

SOURCES = ["indexer.hip", "tokens.hip", "attention.hip", "attention_mla.hip", "attention_d128.hip",
           "hils.hip", "probe.hip", "capi.cpp"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
    # matrix-core accumulators in VGPRs: the attention kernels keep their
    # resident operands in AGPRs and the accumulators next to the VALU
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libhisa_sanitize.so")
# host-side only: each sanitizer flag applies to the host compilation
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host",
                  "-fno-sanitize-recover=undefined"]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime matching hipcc's host compiler."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang ASan runtime not found")
    return cands[-1]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + lang + COMMON_FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o",
                                                           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(jobs: int = 8, verbose: bool = True) -> str:
    """The host-sanitized test copy of the library (see the module notes)."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, SANITIZE_DIR, SANITIZE_FLAGS), SOURCES))
    tmp = SANITIZE_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address",
           "-fsanitize=undefined", "-shared-libsan", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SANITIZE_LIB)
    if verbose:
        print(f"built {SANITIZE_LIB}")
    return SANITIZE_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args(argv)
    if a.sanitize:
        build_sanitized(a.jobs)
    else:
        build(a.jobs)


if __name__ == "__main__":
    sys.exit(main())
