"""The attention blocks' work-item mapping (wf_internal.h: xcd_work_item,
xcd_run_item) is a permutation of the work list for the five workload
shapes and thousands of random group layouts: every (head, query group,
query tile) is computed exactly once.  The check is host C++ built from the
library's own header (hipcc, host code only; no GPU)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "chunk_wise_causal_amd", "csrc")


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def test_work_item_mapping_is_a_permutation(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "work_map_check")
    build = subprocess.run(
        [cc, "-O1", "-std=c++17", "--cuda-host-only", f"-I{CSRC}",
         os.path.join(HERE, "csrc", "work_map_check.cpp"), "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok:"), run.stdout
