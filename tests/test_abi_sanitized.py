"""The C ABI layer (mla_api.cpp) built for the host with the address and
undefined-behaviour sanitizers, against stand-ins for the HIP runtime calls
and kernel launchers (tests/abi_host/stubs.cpp), and driven through every
entry point with valid and invalid arguments (tests/abi_host/driver.cpp).
No GPU is needed; any sanitizer report or wrong status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "abi_host")
CSRC = os.path.join(ROOT, "head_latent_attention_absorbed_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_host"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "mla_api.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr[-4000:]
    assert "abi host checks passed" in run.stdout
