"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the planner (spec validation, SegmentPageTable, page allocation, work lists,
growth) built host-only with g++ -fsanitize=address,undefined, then the planner,
validation, append and random-spec CPU tests run against that build in a child
process. Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_segmentpagetable_amd", "csrc")

# CPU tests that call only the planner's entry points (the others need the kernels'
# entry points, which this build does not contain)
KEEP = "not call_validation and not exports and not select_and_transfer and " \
       "not decode_without_items and not append_errors"


def test_planner_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime")
    lib = tmp_path / "libsegpaged_planner_san.so"
    build = subprocess.run(
        [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "planner.cpp"),
         "-o", str(lib)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ)
    env["SEGPAGED_LIB"] = str(lib)
    env["LD_PRELOAD"] = asan  # the runtime must come first; python itself is not instrumented
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
         "-k", KEEP, "tests/test_planner.py", "tests/test_append.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    # the child really ran the sanitized build, and ran the tests
    assert " passed" in run.stdout and "deselected" in run.stdout, out[-2000:]
