"""Address and undefined-behaviour sanitizer builds of the host code (CPU only):

- the fp64 oracle (gcc, -fsanitize=address,undefined) on a small varlen batch with empty,
  1-, 2- and 17-token sequences;
- the C ABI's argument checks (kda_api.hip, host side built with the sanitizers through
  -Xarch_host; the kernels are not part of it) with every rejection path and the empty
  calls, linked with launchers that count as a failure if any call reaches them.

Each driver exits 0 and prints "ok"; a sanitizer report makes it exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "kda_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "2"})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_checks_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    host = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer",
                 "-fno-sanitize-recover=all"):
        host += ["-Xarch_host", flag]
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gated_delta_rule_31_amd", "csrc"),
           os.path.join(ROOT, "gated_delta_rule_31_amd", "csrc", "kda_api.hip"), os.path.join(HERE, "abi_driver.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    # (the HIP runtime's own allocations at exit are not this code's: no leak check)
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
