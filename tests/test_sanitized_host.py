"""The CPU oracle and the host side of the HIP library, built once with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no GPU code is
instrumented) and driven through their edge cases (tests/sanitize/). A
sanitizer report aborts the driver, so a zero exit status means no
out-of-bounds access, use after free or undefined behaviour on those paths."""

import os
import subprocess

import pytest
import torch

from gated_delta_rule_98_amd import build as gpu_build
from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", *SAN, oracle_build.SRC,
                    os.path.join(HERE, "sanitize", "oracle_driver.c"), "-o", exe, "-lm", "-lpthread"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="hands fake device addresses to the library")
def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    host_san = [x for flag in SAN for x in ("-Xarch_host", flag)]
    cmd = [gpu_build.HIPCC, f"--offload-arch={gpu_build.ARCH}", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, f"-I{gpu_build.INCLUDE}",
           *gpu_build.SOURCES, os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi driver: ok" in r.stdout
