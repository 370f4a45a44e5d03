"""The library's host code (allocators and planner) under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/fuzz_host.cpp drives random operation sequences through the C
API of alloc.cpp and plan.cpp, built here with g++ and the sanitizers, and
checks the allocator invariants of the "Paged KV cache" page (Code: append
with copy-on-write, fork, release) and of the GraniKV HOT pool (Section 3.2)
after every operation, plus the planner's documented caps.  Any sanitizer
report aborts the program; a broken invariant exits 1 naming it.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "shared_prefix_paged_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("sanitize") / "fuzz_host")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "alloc.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "fuzz_host.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_allocators_and_planner_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, str(seed), "150"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-4000:]
