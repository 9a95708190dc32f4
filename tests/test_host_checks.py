"""Host code under the sanitizers, on the CPU.

* The library's HIP-free host logic (the stand-in patcher of the session
  drivers and the debug build's pass-descriptor checks) is built into a small
  driver with AddressSanitizer and UndefinedBehaviorSanitizer (g++, no
  recovery) and checked: the patcher against the oracle's segmentation
  (pytorch.kr Fast-BLT summary, "pre-training and setup" for the patch
  rule's role, "BLT-D attention mask" for the targets), also when a copy
  continues it as the draft rounds do; the descriptor checker accepts the layouts the entry points
  build and names each planted violation.
* The host-sanitized library build (libblt_asan.so) loads with the clang
  ASan runtime preloaded and its argument validation runs clean.
"""
import json
import os
import random
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import patcher  # noqa: E402

HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("host") / "host_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Werror", *SAN,
                    os.path.join(HOST, "host_check.cpp"), "-o", exe], check=True)
    return exe


def run_driver(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


def parse_state(line):
    f = line.split()
    assert f[0] == "S"
    pe = [tuple(map(int, t.split(":"))) for t in f[3:]]
    return int(f[1]), int(f[2]), [p for p, _ in pe], [bool(e) for _, e in pe]


def oracle_state(x, lens, salt):
    p, e = patcher.segment(x, lens, salt)
    # running patch length and newest complete patch after the last byte
    cur = 0
    for i in range(len(x)):
        cur = 1 if i == 0 or e[i - 1] else cur + 1
    return cur, patcher.last_complete_patch(p, e), list(map(int, p)), list(map(bool, e))


def test_patcher_matches_oracle_under_sanitizers(driver):
    rng = random.Random(20261203)
    cases, expect = [], []
    for _ in range(200):
        lens = [1] + [rng.randint(1, 8) for _ in range(rng.randint(0, 6))]
        n_prompt = sum(lens)
        x = [rng.randrange(256) for _ in range(n_prompt + rng.randint(0, 40))]
        salt = rng.getrandbits(64)
        t = rng.randint(n_prompt, len(x))
        cases.append(" ".join(map(str, ["P", salt, len(lens), *lens, len(x), *x, t])))
        full = oracle_state(x, lens, salt)
        expect.append((oracle_state(x[:n_prompt], lens, salt), full, full))
    out = run_driver(driver, cases)
    assert len(out) == 3 * len(cases)
    for k, exp in enumerate(expect):
        for j in range(3):
            assert parse_state(out[3 * k + j]) == exp[j], (cases[k], j)


# limits: max_batch 4, max_ctx 512, max_latents 64, max_rows 64, block_tok 4 x 8
LIMITS = [4, 512, 64, 64, 32]


def block_step_layout(starts, n_app, B, causal=False):
    """Rows and sequences as the block entry point lays them out: per
    sequence (slot b) n_app appended clean rows, then B block rows."""
    rows, seqs = [], []
    for b, (s0, na) in enumerate(zip(starts, n_app)):
        row0, end = len(rows), s0 + na + B
        for j in range(na):
            rows.append([b, s0 + j, 65 + j, 0, 3, s0 + j + 1, -1, 0, -1, 0])
        for j in range(B):
            pos = s0 + na + j
            rows.append([b, pos, -1, b * B + j, 5, pos + 1 if causal else end, b * B + j, 0, -1, 0])
        seqs.append([b, row0, na + B, end, b * B, row0 + na, B, b, 0])
    return rows, seqs


def desc_line(rows, seqs, limits=LIMITS):
    return " ".join(map(str, ["D", *limits, len(rows), *[v for r in rows for v in r],
                              len(seqs), *[v for q in seqs for v in q]]))


def test_descriptor_checks_accept_valid_layouts_and_name_each_violation(driver):
    import copy
    ok_cases = [block_step_layout([10, 20], [2, 0], 4), block_step_layout([0, 7, 9], [1, 1, 3], 8, True),
                block_step_layout([500], [0], 8)]
    # clean rows only (the row-append entry point) and an empty pass
    ok_cases.append(([[1, p, 66, 0, 2, p + 1, 0, 0, -1, 0] for p in range(3, 6)], [[1, 0, 3, 6, -1, -1, 0, 1, 0]]))
    ok_cases.append(([], []))
    base_rows, base_seqs = block_step_layout([10, 20], [2, 1], 4)
    R, S = 0, 1
    muts = [  # (rows or seqs, index, field, value, expected message fragment)
        (R, 0, 0, 4, "row slot"), (R, 0, 1, -1, "row position"), (R, 2, 1, 512, "row position"),
        (R, 0, 5, 10, "row kend"), (R, 3, 5, 513, "row kend"), (R, 1, 4, 64, "row latent"),
        (R, 1, 4, -1, "row latent"), (R, 0, 2, 257, "row token"), (R, 0, 2, -3, "row token"),
        (R, 2, 3, -1, "token source index"), (R, 2, 3, 32, "block index"), (R, 0, 6, -2, "output index"),
        (R, 0, 8, -2, "draw number"), (R, 0, 7, 2, "flag"), (R, 0, 9, 3, "flag"),
        (R, 3, 1, 12, "two rows write one cache row"), (R, 0, 0, 1, "slot differs"),
        (R, 0, 7, 1, "attention kernel differs"),
        (S, 0, 0, -1, "sequence slot"), (S, 0, 7, 4, "batch index"), (S, 1, 2, 9, "rows outside the pass"),
        (S, 0, 3, 15, "kmax"), (S, 0, 6, 7, "block rows outside"), (S, 0, 5, 3, "block rows outside"),
        (S, 1, 4, 30, "beyond block_tok"), (S, 0, 6, -1, "count negative"), (S, 0, 8, 2, "flag"),
        (S, 1, 1, 5, "row in two sequences"),
    ]
    lines = [desc_line(r, s) for r, s in ok_cases]
    for which, i, f, v, _ in muts:
        rows, seqs = copy.deepcopy(base_rows), copy.deepcopy(base_seqs)
        (rows if which == R else seqs)[i][f] = v
        lines.append(desc_line(rows, seqs))
    lines.append(desc_line(ok_cases[3][0], [[1, 0, 2, 5, -1, -1, 0, 1, 0]]))  # row 2 in no sequence
    lines.append(desc_line(base_rows, base_seqs, [4, 512, 64, 8, 32]))   # 11 rows > max_rows
    out = run_driver(driver, lines)
    assert out[:len(ok_cases)] == ["ok"] * len(ok_cases), out[:len(ok_cases)]
    for (which, i, f, v, frag), got in zip(muts, out[len(ok_cases):]):
        assert got.startswith("debug bounds:") and frag in got, ((which, i, f, v), got)
    assert "row in no sequence" in out[-2]
    assert "row count" in out[-1]


def test_sanitized_library_loads_and_validates_arguments():
    from block_diffusion_byte_amd import build as bld
    lib = os.path.join(ROOT, "block_diffusion_byte_amd", "libblt_asan.so")
    if not os.path.exists(lib):
        bld.build(variant="asan")
    try:
        rt = bld.asan_preload()
    except FileNotFoundError:
        pytest.skip("g++ ASan runtime not installed")
    code = r"""
import ctypes as C, json, sys
sys.path.insert(0, %r)
import block_diffusion_byte_amd as b
L = b.lib()
assert b.LIB_PATH.endswith("libblt_asan.so"), b.LIB_PATH
res = {}
res["bw"] = list(b.blt_bw_model(1000, 100, 2, 160_000_000, 19_000_000, 1_280_000_000))
# a context with a bad configuration is refused before any device call
res["create_null"] = L.blt_create(None, None, None, None)
res["state_size_null"] = L.blt_state_size(None, None, None)
# C++ exceptions thrown inside other libraries of the process (torch's
# device probing with no device visible) pass through the sanitizer runtime
import torch
try:
    torch.zeros(1).to("cuda:0")
except RuntimeError:
    pass
print(json.dumps(res))
""" % ROOT
    env = dict(os.environ, BLT_LIB="asan", LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["create_null"] == -1 and res["state_size_null"] == -1
    from oracle import proxy
    assert res["bw"][0] == proxy.proxy_bytes(1000, 100, 160_000_000, 19_000_000, 1_280_000_000)
    assert np.isclose(res["bw"][1], float(proxy.proxy_gb_per_seq(1000, 100, 2, 160_000_000, 19_000_000,
                                                                   1_280_000_000)), rtol=1e-12)
