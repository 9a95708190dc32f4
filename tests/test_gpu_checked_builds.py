"""The native decode sessions through the checked library builds, on the GPU.

The bounds-checking build (libblt_debug.so: every staged pass descriptor is
checked against the context's geometry) and the host-sanitized build
(libblt_asan.so: that build's host code compiled by g++ with AddressSanitizer
and UndefinedBehaviorSanitizer) run, from a plain C++ driver over the C-ABI
(tests/host/session_driver.cpp, built with the same sanitizers for the
sanitized library), the sessions the release build runs here through the
Python binding: greedy, BLT-D (threshold, entropy bound, device-resident
blocks), BLT-S, BLT-DV (one step and sampled) and a bfloat16 block pass on
the MFMA path.  Every session must complete without a check or sanitizer
report and give the release build's bytes and counters (pytorch.kr Fast-BLT
summary, "BLT-D inference" and "BLT-S and BLT-DV": the policies driven).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests", "host"))

import sessions  # noqa: E402

pytestmark = pytest.mark.gpu

PKG = os.path.join(ROOT, "block_diffusion_byte_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def release_results():
    import block_diffusion_byte_amd as blt
    assert blt.LIB_PATH.endswith("libblt.so"), blt.LIB_PATH
    return sessions.run_all()


@pytest.fixture(scope="module")
def cases(tmp_path_factory):
    return sessions.write_cases(str(tmp_path_factory.mktemp("cases")))


def run_variant(variant, cases, tmp_path):
    from block_diffusion_byte_amd import build as bld
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    if not os.path.exists(os.path.join(PKG, f"libblt_{variant}.so")):
        bld.build(variant=variant)
    exe = str(tmp_path / f"driver_{variant}")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{bld.ROCM}/include",
                    *(SAN if variant == "asan" else []), os.path.join(ROOT, "tests", "host", "session_driver.cpp"),
                    f"-L{PKG}", f"-lblt_{variant}", f"-L{bld.ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}",
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    got = {}
    for d, names in cases:
        print(f"libblt_{variant}.so: {names}", flush=True)
        r = subprocess.run([exe, d], capture_output=True, text=True, timeout=600, env=env)
        assert r.returncode == 0, r.stderr[-6000:]
        for bad in ("AddressSanitizer", "runtime error:", "debug bounds:"):
            assert bad not in r.stderr, r.stderr[-6000:]
        got.update(sessions.parse_driver(r.stdout, names))
    return got


def test_bounds_checked_build_runs_every_session_like_release(release_results, cases, tmp_path):
    assert run_variant("debug", cases, tmp_path) == release_results


def test_host_sanitized_build_runs_every_session_like_release(release_results, cases, tmp_path):
    assert run_variant("asan", cases, tmp_path) == release_results
