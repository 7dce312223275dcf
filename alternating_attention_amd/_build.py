"""Builds libvga.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvga.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["vga_api.cpp", "flash_attn.hip", "sga_gather.hip", "register_rows.hip",
           "proj_gemm.hip"]

# Packed fp32 VALU instructions stay disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libvga.so (always rebuilds)."""
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host code built with AddressSanitizer and UBSan for CPU-side checks of the
# argument validation, workspace layouts and schedules (the device code is
# compiled as usual: every sanitizer flag is host-only).  The library links
# the shared clang sanitizer runtime, which the process that loads it must
# preload (sanitizer_runtime()).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(ROOT, "_build", "asan", "libvga.so")


def sanitizer_runtime() -> str:
    """Path of the shared clang AddressSanitizer runtime to LD_PRELOAD."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """libvga.so with sanitized host code, into _build/asan/ (CPU tests only)."""
    build_dir = os.path.join(ROOT, "_build", "asan")
    os.makedirs(build_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = ([HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
               + DEVICE_FLAGS + SANITIZE_HOST)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = ([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", SANITIZED_LIB] + objs
           + ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-shared-libasan"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    if verbose:
        print("built", SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    build(verbose=True)
