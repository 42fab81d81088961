"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/csrc/abi_sanitize_check.cpp calls every entry point of include/wf.h
with arguments that break its contract (and with documented no-op
arguments) and checks each status code and message.  It is linked against
the library's host code (api.cpp, compiled host-only) with the launch
functions and the HIP runtime calls stubbed to abort, so the checks run with
no GPU and no HIP runtime, and any out-of-bounds access, use of freed
memory, signed overflow or misaligned access on those paths stops the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "chunk_wise_causal_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["address", "undefined"]


def _tool(*names):
    for n in names:
        p = os.path.join(ROCM, *n.split("/"))
        if os.path.exists(p):
            return p
    return None


def test_entry_point_checks_under_sanitizers(tmp_path):
    hipcc = _tool("bin/hipcc")
    clang = _tool("llvm/bin/clang++")
    if hipcc is None or clang is None:
        pytest.skip("hipcc / clang++ not available")
    # host-only objects; each -fsanitize= applies to the host pass only
    cflags = ["-O1", "-g", "-std=c++17", "--cuda-host-only", "-x", "hip", f"-I{INCLUDE}",
              f"-I{CSRC}", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    for s in SAN:
        cflags += ["-Xarch_host", f"-fsanitize={s}"]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "csrc", "abi_sanitize_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *cflags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_sanitize_check")
    r = subprocess.run([clang, "-fsanitize=" + ",".join(SAN), *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the environment is kept as it is; a preloaded library ahead of the
    # sanitizer runtime is tolerated rather than removed
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stdout + run.stderr[-4000:]
    assert run.stdout.startswith("ok "), run.stdout
    assert "runtime error" not in run.stderr, run.stderr[-4000:]
    assert int(run.stdout.split()[1]) == 33
