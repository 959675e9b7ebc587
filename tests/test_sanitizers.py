"""Host builds with the address and undefined-behaviour sanitizers (CPU only):
the fp64 oracle driven through every input kind, form, mask and ragged
offsets (tests/sanitize/oracle_checks.c), and the C ABI's argument validation
(tests/sanitize/abi_checks.cpp, linked against the library's host sources with
stand-ins for the kernel launchers; the sanitizers apply to host code only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "linear_attention_rnn_finch_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "all checks passed" in out and "runtime error" not in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                    os.path.join(ROOT, "oracle", "wkv_oracle.c"), os.path.join(HERE, "oracle_checks.c"),
                    "-lm", "-o", exe], check=True, capture_output=True, timeout=300)
    _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_host_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "abi_checks.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
           os.path.join(CSRC, "wkv_api.cpp"), os.path.join(CSRC, "wkv_noalloc.hip"),
           os.path.join(CSRC, "wkv_query.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    _run(exe)
