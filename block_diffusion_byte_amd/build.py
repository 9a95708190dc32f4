"""Build libblt.so (HIP kernels + C-ABI + native decode drivers) for gfx950.

Usage: python -m block_diffusion_byte_amd.build [--variant release|debug|asan]

Variants (the device code is the same in all three):
  release  libblt.so        -O3
  debug    libblt_debug.so  host code -O1 -g with BLT_DEBUG_BOUNDS: every
                            staged pass descriptor is checked against the
                            context's geometry before it goes to the device
  asan     libblt_asan.so   the debug build's host code compiled by g++ with
                            AddressSanitizer and UndefinedBehaviorSanitizer
                            (host code only; load it with g++'s ASan runtime
                            preloaded)
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["kernels.hip", "blt_api.cpp", "session.cpp"]
ARCH = os.environ.get("BLT_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GXX = os.environ.get("CXX_HOST", "g++")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# Packed fp32 instructions are kept out of generated code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
# the host sources hold no device code, so g++ compiles them for the
# sanitized build (its ASan runtime leaves the HIP runtime's allocations alone)
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
VARIANTS = {
    "release": ("libblt.so", ["-O3"], []),
    "debug": ("libblt_debug.so", ["-O1", "-g", "-DBLT_DEBUG_BOUNDS"], []),
    "asan": ("libblt_asan.so", ["-O1", "-g", "-DBLT_DEBUG_BOUNDS"], SANITIZE),
}


def asan_preload() -> str:
    """LD_PRELOAD value for a process that uses libblt_asan.so: g++'s ASan
    runtime, then libstdc++ (so the runtime finds the real __cxa_throw for
    the C++ exceptions other libraries of the process throw)."""
    paths = []
    for lib in ("libasan.so", "libstdc++.so"):
        r = subprocess.run([GXX, f"-print-file-name={lib}"], capture_output=True, text=True)
        path = r.stdout.strip()
        if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
            raise FileNotFoundError(f"g++'s {lib} not found")
        paths.append(os.path.realpath(path))
    return ":".join(paths)


def _compile(src, obj, flags, verbose, gxx=False):
    if gxx:
        cmd = [GXX, *COMMON, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *flags]
    else:
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *flags]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    if verbose:
        msgs = [m for m in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in m]
        if msgs:
            print("\n".join(msgs))


def build(verbose: bool = False, variant: str = "release") -> str:
    name, opt, extra = VARIANTS[variant]
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src.endswith(".hip") and variant != "release":
            # the kernels and their launchers are the release object's
            obj = os.path.join(objdir, src + ".o")
            if not os.path.exists(obj):
                _compile(src, obj, VARIANTS["release"][1], verbose)
        else:
            obj = os.path.join(objdir, f"{src}.{variant}.o" if variant != "release" else src + ".o")
            _compile(src, obj, opt + extra, verbose, gxx=variant == "asan")
        objs.append(obj)
    out = os.path.join(HERE, name)
    tmp = out + ".tmp"
    if variant == "asan":
        cmd = [GXX, "-shared", *SANITIZE, *objs, f"-L{ROCM}/lib", "-lamdhip64", "-o", tmp]
    else:
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link of {name} failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="release")
    print(build(verbose=True, variant=ap.parse_args().variant))
