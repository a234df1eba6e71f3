"""The host table code (binary128 decision points and levels, the per-alpha
memo) built with g++ under AddressSanitizer + UBSan and under ThreadSanitizer,
driven from four threads over many alphas and every code width; any sanitizer
report fails the run.  Host code only: no GPU, no HIP kernels."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a16_linear_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                                   ["-fsanitize=thread"]], ids=["asan_ubsan", "tsan"])
def test_host_tables_under_sanitizers(tmp_path, flags):
    exe = str(tmp_path / "drv")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
            "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC] + flags +
           [os.path.join(ROOT, "tests", "host", "tables_driver.cpp"),
            os.path.join(CSRC, "tables.cpp"), "-lquadmath", "-pthread", "-o", exe])
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad=0" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr
