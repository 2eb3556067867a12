"""The host slot table's tests under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The planner (libmoe_planner.so, the same sources as the GPU library's host slot table) is
rebuilt with g++ -fsanitize=address,undefined, and the planner-against-oracle tests run
against that build in a child process with the ASan runtime preloaded; any invalid access,
leak-free or not, or undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build_planner_sanitized(out_path):
    """The host slot table alone (the planner sources of the library), built with g++ and the
    address and undefined-behaviour sanitizers, no HIP."""
    from expert_offload_lru_amd import build
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-Wall", "-I" + build.INCLUDE, "-I" + build.CSRC,
           "-o", out_path] + [os.path.join(build.CSRC, n) for n in build.PLANNER_SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out_path


@pytest.mark.slow
def test_planner_tests_pass_under_asan_and_ubsan(tmp_path):
    lib = build_planner_sanitized(str(tmp_path / "libmoe_planner_san.so"))
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["g++", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan) and os.path.exists(ubsan), (asan, ubsan)
    env = dict(os.environ, MOE_PLANNER_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_planner_vs_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
