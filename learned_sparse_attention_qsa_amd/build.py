"""Build libqsa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m learned_sparse_attention_qsa_amd.build        # or build()

Outputs learned_sparse_attention_qsa_amd/lib/libqsa.so.  Every call rebuilds.
build_sanitized() builds lib/libqsa_san.so, the same library with its host
code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (device
code unchanged), for the CPU tests of the C ABI's argument checking.
build_debug() builds lib/libqsa_debug.so with QSA_DEBUG: the kernels' guards
on caller-supplied values also count what they catch (qsa_debug_guard_hits).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(LIBDIR, "libqsa.so")
SAN_LIB = os.path.join(LIBDIR, "libqsa_san.so")
SAN_OBJDIR = os.path.join(PKG, "_build", "san")
DEBUG_LIB = os.path.join(LIBDIR, "libqsa_debug.so")
DEBUG_OBJDIR = os.path.join(PKG, "_build", "debug")
# host-side sanitizers only: each flag behind -Xarch_host
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]
SOURCES = ["compress.hip", "expand.hip", "topk.hip", "attend.hip", "ceilings.hip", "noalloc.hip",
           "backward.hip",
           "api.cpp"]
# The stream scorer's MFMA results are read by a vector epilogue every tile:
# the VGPR form of MFMA keeps them out of accumulation registers (no
# v_accvgpr_read per value).
FILE_FLAGS = {"topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, san: bool = False, debug: bool = False) -> str:
    objdir = SAN_OBJDIR if san else (DEBUG_OBJDIR if debug else OBJDIR)
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    extra = SAN_FLAGS if san else (["-DQSA_DEBUG"] if debug else [])
    cmd = [_hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-O2" if not san else "-O1", f"--offload-arch={ARCH}", "-fPIC",
               "-std=c++17", *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(SAN_OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, san=True), SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan",
           *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build_debug(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(DEBUG_OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug=True), SOURCES))
    tmp = DEBUG_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DEBUG_LIB)
    if verbose:
        print(f"built {DEBUG_LIB}")
    return DEBUG_LIB


def sanitizer_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into a
    process that loads libqsa_san.so)."""
    hip_bin = os.path.dirname(os.path.realpath(_hipcc()))
    for cxx in (os.path.join(hip_bin, "..", "llvm", "bin", "clang++"),
                "/opt/rocm/llvm/bin/clang++", "clang++"):
        try:
            r = subprocess.run([cxx, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
        except OSError:
            continue
        path = r.stdout.strip()
        if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
            return path
    raise RuntimeError("AddressSanitizer runtime not found")


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
