"""Build libmha.so in-tree with hipcc for gfx950 (MI355X).

Usage: python -m transformer_scaled_dot_mha_amd.build [-v]
Objects go to _build/ at the repository root; the library is written next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import glob
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmha.so")
BUILD_INFO = os.path.join(HERE, "libmha.build.json")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for device code: the compiler would
# otherwise pair independent fp32 operations into v_pk_* instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmha.so")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; drop that warning
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip()
             and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    # the toolchain that built the library, for the bench record (read there
    # without running the compiler from a process that uses the GPU)
    ver = subprocess.run([_hipcc(), "--version"], capture_output=True, text=True).stdout
    info = {"hipcc_version": ver.strip().splitlines(), "arch": ARCH, "flags": COMMON + DEVICE_FLAGS}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)
    return LIB


ASAN_LIB = os.path.join(OBJDIR, "libmha_host_asan.so")


def build_host_asan(verbose: bool = False) -> str:
    """The C front end (mha_api.cpp: validation, workspace layout, status and
    error text) built for the host with AddressSanitizer, its kernel launchers
    replaced by stubs (tests/asan/launch_stubs.cpp). CPU only: no device code."""
    os.makedirs(OBJDIR, exist_ok=True)
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, "mha_api.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", ASAN_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("host ASan build failed:\n" + r.stdout + r.stderr)
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
