"""The oracle and the library's host-side argument validation, each built
with AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

The oracle driver (tests/sanitize/oracle_driver.c) calls every oracle entry
point over small ragged and multi-tile tensors with every option; the ABI
driver (tests/sanitize/abi_driver.c, in C like the ABI's callers) calls every
entry point of include/nvfp4.h with arguments that must be rejected before any
launch, including enum values outside their enumerators, sizes whose products
overflow and row offsets whose element indices would.  Only host code is
instrumented (the GPU code of the library is built as usual and never runs).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"), "-o", str(exe),
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-lm", "-pthread"])
    res = _run([str(exe)], env=ENV, timeout=300)
    assert "all calls clean" in res.stdout
    assert "runtime error" not in res.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_abi_validation_under_address_and_undefined_sanitizers(tmp_path):
    obj = tmp_path / "abi_driver.o"
    exe = tmp_path / "abi_san"
    inc = os.path.join(ROOT, "include")
    _run([CLANG, "-c", "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-I", inc, "-o", str(obj),
          os.path.join(SAN, "abi_driver.c")])
    csrc = os.path.join(ROOT, "nvfp4_block_quantization_amd", "csrc")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san, "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, "-o", str(exe), str(obj),
          "-x", "hip", os.path.join(csrc, "nvfp4.hip"), os.path.join(csrc, "gemm.hip")])
    res = _run([str(exe)], env=ENV, timeout=300)
    assert "all rejections clean" in res.stdout
    assert "runtime error" not in res.stderr
