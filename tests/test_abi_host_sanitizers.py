"""The C ABI front end (gptq_abi.cpp: argument checks, workspace sizing,
launch sequencing) built for the host alone with the address and
undefined-behaviour sanitizers, against stand-in launchers, and driven
through every entry point's accepted and rejected argument sets
(tests/host_abi).  No GPU: the device code is not compiled here."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_abi")
CSRC = os.path.join(ROOT, "post_weight_quantization_syrk_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


def test_abi_front_end_under_host_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "drive_abi")
    flags = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", f"-I{CSRC}",
             f"-I{os.path.join(ROOT, 'include')}"]
    srcs = [os.path.join(CSRC, "gptq_abi.cpp"), os.path.join(HERE, "stub_launchers.cpp"),
            os.path.join(HERE, "drive_abi.cpp")]
    r = subprocess.run([cxx, *flags, *srcs, "-o", exe], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " 0 failed" in r.stdout
