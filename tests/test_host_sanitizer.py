"""The library's host code (include/vap.h's entry points in csrc/api.cpp) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU.

tests/host_check/check_api.cpp calls every entry point at its extremes (8192 sequences, 64 query
rows per sequence, 32768-token contexts; verification batches up to 2^22 sequences, k up to 64,
vocabularies up to 2^20, trees of 64 nodes) with the default, minimum and intermediate
workspaces, plus argument errors.  tests/host_check/stubs.cpp stands in for the HIP runtime and
the kernel launchers: each launcher checks that every region the host code carved lies inside
the workspace the call was given.  The host code is compiled for the host only (no device code,
no HIP runtime linked), so this runs without a GPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["verify_attention_paged_amd/csrc/api.cpp", "tests/host_check/stubs.cpp", "tests/host_check/check_api.cpp"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # host pass only; each sanitizer flag is passed to the host compilation explicitly
        cmd = [HIPCC, "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "verify_attention_paged_amd", "csrc"),
               "-c", os.path.join(ROOT, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "check_api")
    res = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert " 0 carving violations, 0 failures" in run.stdout
