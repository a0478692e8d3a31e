"""Schedule generation, binding and work-list layout (the C++ host code of the
library) under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/host_check/host_check.cpp is compiled with g++ together with plan.cpp
and bind.cpp (no HIP code) and checks the invariants the kernels rely on for a
grid of shapes: hazard-free schedules, every byte of every row bound once,
work-list pieces inside one column group of their owner's list, in step
order, with correct wave masks, and runs of at most RUN_MAX one-tile pieces of
one step with no common destination bytes.

A second build (-O2, no sanitizers) also executes a sample of the work lists
symbolically, as the forwarding and the plain variants of the row kernel take
them: the same memory as running the items step by step, and no unit that one
work group writes touched by another in the same launch.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "collective_communication_algorithms_amd", "csrc")


SOURCES = [os.path.join(ROOT, "tests", "host_check", "host_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "bind.cpp"), os.path.join(CSRC, "colprog.cpp")]
INCLUDES = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _build_and_run(tmp_path, flags, args, env=None):
    exe = str(tmp_path / "host_check")
    r = subprocess.run(["g++", "-std=c++17", *flags, *INCLUDES, *SOURCES, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert r.stdout.strip().endswith("ok"), r.stdout[-2000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    _build_and_run(tmp_path, ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                              "-fno-omit-frame-pointer"], ["--exec=none"], env)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_work_lists_execute_like_the_steps(tmp_path):
    out = _build_and_run(tmp_path, ["-O2"], ["--exec=sample"])
    assert " 0 list executions" not in out and " 0 skipped stores" not in out, out
