"""Compile the HIP sources into the in-tree shared library ``libpa.so``.

Every source is compiled for gfx950 with hipcc; packed fp32 instructions are
disabled for device code. Objects go to ``_build/`` (not committed); the
library is written next to this file and replaced atomically.
"""

from __future__ import annotations

import os
import shlex
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")
SOURCES = ["attention.hip", "balanced.hip", "prefill.hip", "write_kv.hip", "lse_merge.hip",
           "block_manager.cpp",
           "pa_api.cpp"]
# the benchmark's HBM read ceilings (include/pa_probe.h), a library of its own
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libpa_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpa.so")
    return path


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs: with AGPR accumulators the prefill
        # kernel's conditional rescale made the compiler mirror all of them
        # through VGPRs on every block
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib_path: str) -> None:
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib_path)} failed:\n{res.stdout}\n"
                           f"{res.stderr}")
    os.replace(tmp, lib_path)


def build(jobs: int = 4, extra_flags=(), lib_path: str = LIB_PATH,
          build_dir: str = BUILD_DIR) -> str:
    """Compile and link; ``extra_flags`` (e.g. ``-DPA_KV_DEPTH=3``) override
    the compile-time tunables of the kernels."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(lambda src: _compile(src, build_dir, tuple(extra_flags)), SOURCES))
    _link(objs, lib_path)
    return lib_path


# Host code checked under sanitizers on the CPU: the block manager and the C
# API's validation and sizing. Host-only instrumentation (each flag behind
# -Xarch_host): device code is compiled as usual.
HOST_SANITIZED_SOURCES = ("block_manager.cpp", "pa_api.cpp")
HOST_SANITIZE_FLAGS = shlex.split(
    "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
    "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer -O1")
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
HOST_CHECKS = os.path.join(ROOT, "tests", "c_abi", "host_checks.cpp")


def build_host_sanitized(build_dir: str = SANITIZE_DIR) -> str:
    """libpa with AddressSanitizer and UndefinedBehaviorSanitizer on the host
    code of HOST_SANITIZED_SOURCES (the kernels' sources as usual), and the
    CPU program tests/c_abi/host_checks.cpp linked against it with the
    sanitizer runtimes. Returns the program's path; running it needs no GPU."""
    os.makedirs(build_dir, exist_ok=True)
    objs = [_compile(src, build_dir, tuple(HOST_SANITIZE_FLAGS)
                     if src in HOST_SANITIZED_SOURCES else ())
            for src in SOURCES]
    lib = os.path.join(build_dir, "libpa_host_sanitized.so")
    _link(objs, lib)
    exe = os.path.join(build_dir, "host_checks")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin",
                         "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    cmd = [clang, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), HOST_CHECKS, "-o", exe,
           lib, "-Wl,-rpath," + build_dir]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking host_checks failed:\n{res.stdout}\n{res.stderr}")
    return exe


def build_probe(build_dir: str = BUILD_DIR) -> str:
    """The benchmark's read-ceiling library, libpa_probe.so."""
    os.makedirs(build_dir, exist_ok=True)
    _link([_compile(src, build_dir) for src in PROBE_SOURCES], PROBE_LIB_PATH)
    return PROBE_LIB_PATH


if __name__ == "__main__":
    print(build())
    print(build_probe())
