"""Build libsa.so for gfx950 with hipcc (in-tree; objects under _build/)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsa.so")
SOURCES = ["sa_api.hip", "est_kernels.hip", "attn_kernels.hip", "decode_kernels.hip", "cal_kernels.hip",
           "anchor_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=fast",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         # packed fp32 VALU instructions stay disabled in all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r


# the debug build: the same sources with the kernels' checks of caller data compiled in
DEBUG_LIB = os.path.join(PKG, "libsa_debug.so")
OBJ_DEBUG = os.path.join(OBJ, "debug")


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile libsa.so (and, with debug, libsa_debug.so) in-tree; every source compiles in
    parallel."""
    variants = [(LIB, OBJ, [])] + ([(DEBUG_LIB, OBJ_DEBUG, ["-DSA_DEBUG"])] if debug else [])
    cmds, links = [], []
    for lib, obj_dir, extra in variants:
        os.makedirs(obj_dir, exist_ok=True)
        objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds += [[HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", o]
                 for s, o in zip(SOURCES, objs)]
        links.append((lib, objs))
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 8)) as pool:
        list(pool.map(_run, cmds))
    for lib, objs in links:
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


SAN_LIB = os.path.join(OBJ, "libsa_hostsan.so")
# host-side sanitizers for the C ABI's validation code: each -fsanitize= goes to the host
# pass only (-Xarch_host); the device code is compiled as in the product build
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library needs preloaded."""
    clang = os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang")
    r = _run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"])
    return r.stdout.strip()


def build_host_sanitized(verbose: bool = False) -> str:
    """libsa with the host code of the C ABI (sa_api.hip: argument validation, workspace
    carve-out, launches) built with AddressSanitizer and UndefinedBehaviorSanitizer; the kernel
    objects are those of the product build (build() first).  For CPU tests of the validation
    paths only: loading it needs the ASan runtime preloaded (asan_runtime())."""
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "sa_api.hip"]
    for o in objs:
        if not os.path.exists(o):
            raise RuntimeError("build() the product library first: " + o)
    api_o = os.path.join(OBJ, "sa_api_hostsan.o")
    _run([HIPCC, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "sa_api.hip"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address",
          "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, api_o, *objs])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
