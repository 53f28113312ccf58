"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The host planning code of libmsda (csrc/msda_plan.hpp: descriptor
  validation, packing of the level table and key segments, workspace
  layout, the backward's launch plan) built with g++, run over the C-ABI
  host tests' descriptors, the record envelope's edges (2048 / 2049 / 2052
  segments, 2^24 - 1 and 2^24 queries, 65,534- and 65,535-pixel levels,
  Q = 0, bs = 0) and 100,000 seeded descriptors around the envelope, each
  checked against the invariants the kernels rely on (regions in order and
  large enough, tiles within LDS, grids within range, the accumulation never
  planned without a gradient launch).
* The oracle (oracle/msda_oracle.c) built with gcc, run on tiny and
  degenerate maps with NaN, +-Inf and far off-map locations, at one and four
  threads (results must not depend on the thread count).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]


def _run(cmd, exe, tag):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{tag} failed:\n{r.stdout}\n{r.stderr}"
    assert f"{tag} ok" in r.stdout, r.stdout
    print(r.stdout.strip())


def test_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "scale_deformable_attention_03_amd", "csrc"),
           os.path.join(HERE, "plan_fuzz.cpp"), "-o", exe]
    _run(cmd, exe, "plan_fuzz")


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           os.path.join(ROOT, "oracle", "msda_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe]
    _run(cmd, exe, "oracle_driver")
