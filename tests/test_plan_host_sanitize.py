"""The plan's host-side layout builders under AddressSanitizer and
UndefinedBehaviorSanitizer.

spmm_csr_spmv_amd/csrc/plan_host.cpp holds the row profile, the row bins, the
SELL-C-sigma order, the column-panel and x-window stream layouts, the
phase-swept SpMM copy and the WCSR task table: plain C++ with no HIP.  tests/plan_host_sanitize.cpp
runs them on seeded random matrices and checks their structural invariants;
built here with g++ and the sanitizers, any out-of-bounds access, leak,
overflow, data race visible to the sanitizers or failed check ends the run
with a non-zero status."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_builders_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_host_sanitize")
    csrc = os.path.join(ROOT, "spmm_csr_spmv_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-pthread", "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(HERE, "plan_host_sanitize.cpp"), os.path.join(csrc, "plan_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "40"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok 40 cases" in r.stdout
