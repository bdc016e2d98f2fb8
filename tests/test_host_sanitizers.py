"""The host half of libzl (worklist builder and worklist validation) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, with the same
compiler and flags as the host object of the shipped library, driven by the
randomised checks in host_fuzz.cpp. CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None and shutil.which("c++") is None,
                    reason="no host C++ compiler")
def test_worklist_builder_under_sanitizers(tmp_path):
    exe = tmp_path / "host_fuzz"
    # The sanitizer runtimes are linked statically so that the executable
    # runs under whatever the environment preloads.
    from coalesced_attention_amd.build import HOST_FLAGS, host_cxx
    cmd = [host_cxx(), *HOST_FLAGS, "-g", "-static-libasan", "-static-libubsan",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "coalesced_attention_amd", "csrc"),
           os.path.join(ROOT, "coalesced_attention_amd", "csrc", "zl_host.cpp"),
           os.path.join(ROOT, "tests", "host_fuzz.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe), "400"], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "worklists verified" in res.stdout
