"""The library's host runtime (sv_runtime.cpp) built with g++ against a
host-only stand-in for the HIP API and a toy model in place of the kernels
(tests/host_stub), with the address and undefined-behaviour sanitizers, and
run without a GPU: configuration and buffer checks at create, argument
errors that leave the context untouched, prefill / decode / verify commits
and their histories, rollback, restore, observer-mode state errors, state
cloning through two page tables, batched-verify bookkeeping against
one-at-a-time verifies, the launch count of one forward, and the
no-allocation verify's size limit (SV_ESCRATCH at a 32K context)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "host_stub")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_runtime_logic(tmp_path):
    exe = str(tmp_path / "host_logic_test")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-I", STUB, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "greedy_block_verification_amd", "csrc"), "-o", exe,
           os.path.join(STUB, "host_logic_test.cpp"), os.path.join(STUB, "host_stubs.cpp"),
           os.path.join(ROOT, "greedy_block_verification_amd", "csrc", "sv_runtime.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host logic ok" in run.stdout
