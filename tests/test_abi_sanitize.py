"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the
library sources are compiled with the sanitizers on their host side only (device code as
usual), linked with tests/sanitize/abi_validation.cpp, and run. The driver walks every entry
point's validation with fake device addresses, the descriptor stride and overlap arithmetic
at extreme values, and the workspace sizing of every op at the largest accepted shapes; any
sanitizer report (out-of-bounds access, signed overflow, misaligned access, ...) or wrong
status fails the test."""
import os
import subprocess

import pytest

from block_sparse_attention_top_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.slow
def test_abi_host_code_under_sanitizers(tmp_path):
    cc = B.hipcc()
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [cc, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SANITIZE,
               f"-I{B.INCLUDE}", f"-I{B.CSRC}", "-c", os.path.join(B.CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(obj)
    drv = str(tmp_path / "abi_validation.o")
    cmd = [cc, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", *SANITIZE,
           f"-I{B.INCLUDE}", "-c", os.path.join(HERE, "sanitize", "abi_validation.cpp"), "-o", drv]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    exe = str(tmp_path / "abi_validation")
    cmd = [cc, f"--offload-arch={B.ARCH}", *SANITIZE, drv, *objs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
