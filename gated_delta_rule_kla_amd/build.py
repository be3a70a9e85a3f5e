"""Build libkla.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32
instruction selection disabled and MFMA results kept in architectural VGPRs, and linked into gated_delta_rule_kla_amd/libkla.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkla.so")
SOURCES = ["kla_api.hip", "kla_prep.hip", "kla_scan.hip", "kla_decode.hip", "kla_diag.hip",
           "kla_bwd.hip", "kla_bwd_diag.hip"]
ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in the architectural VGPRs: the kernels feed them straight back
    # into VALU work and other MFMAs, which the AGPR form would route through copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libkla.so")
    return exe


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile all sources and link libkla.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# The same library with AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only
# (the device code is built as usual): the CPU tests drive the C ABI's argument checking and
# error paths through it.  Loading it needs the compiler's ASan runtime first in the process
# (LD_PRELOAD=sanitizer_runtime()).
SAN_FLAGS = [
    *CXXFLAGS, "-g", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that a sanitized build needs preloaded."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm")
    out = subprocess.run([os.path.join(llvm, "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("clang's ASan runtime not found")
    return out


def build_host_sanitized(out_dir: str, jobs: int = 4) -> str:
    """Compile every source with ASan + UBSan on its host code into out_dir/libkla_san.so."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([cc, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host) failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(out_dir, "libkla_san.so")
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs,
                        "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
