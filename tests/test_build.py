"""The build entry point works from a tree that holds sources only: copied without any
built library, `python __graft_entry__.py build` compiles libkda.so and the oracle and
then imports the package (which refuses to import while the library is missing)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_build_from_sources_only(tmp_path):
    dst = tmp_path / "tree"
    skip = shutil.ignore_patterns("*.so", "*.so.tmp*", ".git", "_work", "gpurun_out", "__pycache__", "profiles",
                                  ".pytest_cache")
    shutil.copytree(ROOT, dst, ignore=skip)
    assert not (dst / "gated_delta_rule_31_amd" / "libkda.so").exists()
    r = subprocess.run([sys.executable, "__graft_entry__.py", "build"], cwd=dst, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    assert (dst / "gated_delta_rule_31_amd" / "libkda.so").exists()
    r = subprocess.run([sys.executable, "-c", "import gated_delta_rule_31_amd as k; print(k.LIB_PATH)"], cwd=dst,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == str(dst / "gated_delta_rule_31_amd" / "libkda.so"), r.stderr
