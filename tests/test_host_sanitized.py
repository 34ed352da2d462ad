"""The host control plane (paged_kv_cache_243_amd/csrc/pages_host.cpp) built
on its own with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, and
driven by tests/host_fuzz.cpp: seeded random operations through the public C
functions of include/pagedkv_host.h, valid and invalid ones mixed, with the
header's invariants checked after each (reference counts against the pages in
use, page counts of every sequence, stale handles refused, failing calls
changing nothing, outputs written only within their stated sizes) and the
whole pool free again at the end.  Any sanitizer report or failed check makes
the run exit non-zero.  CPU only; the GPU library is not involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SEEDS = range(12)
STEPS = 4000


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("host_fuzz") / "host_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "paged_kv_cache_243_amd", "csrc"),
           os.path.join(ROOT, "paged_kv_cache_243_amd", "csrc", "pages_host.cpp"),
           os.path.join(ROOT, "tests", "host_fuzz.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("this g++ cannot build with the sanitizers")
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", SEEDS)
def test_host_control_plane_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, str(seed), str(STEPS)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", f"seed {seed}: rc {r.returncode}\n{r.stderr[-4000:]}"
