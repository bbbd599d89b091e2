"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (every entry point on small ragged inputs with junk ids) and the host
side of the C ABI (descriptor checks and workspace planning over a grid of
valid and invalid descriptors, and the argument checks of every compute
entry point).  No GPU code runs; the sanitizers abort on a finding."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def run(cmd, env=None):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env)
    return res.returncode, res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    rc, out = run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                   os.path.join(ROOT, "oracle", "nsa_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                   "-o", exe, "-lm"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    rc, out = run([exe], env)
    assert rc == 0 and "oracle driver ok" in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_asan")
    rc, out = run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                   os.path.join(ROOT, "nsa_selected_block_amd", "csrc", "api.hip"),
                   os.path.join(SAN, "abi_host_driver.cpp"), "-o", exe])
    assert rc == 0, out
    # (the HIP runtime's own start-up allocations are not this library's)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out = run([exe], env)
    assert rc == 0 and "0 failures" in out, out
