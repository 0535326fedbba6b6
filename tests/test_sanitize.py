"""Host-side sanitizer runs (no GPU): the C oracle and the C ABI's argument
validation built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven over edge inputs (tests/sanitize/).  The C ABI is compiled for the
host only, its kernel launchers replaced by stand-ins that count the
launches that validation lets through; no device code is built."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"], ROOT)
    r = _run([exe], ROOT)
    assert "oracle driver clean" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_abi_validation_under_sanitizers(tmp_path):
    host = ["-x", "hip", "--offload-host-only", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-O1", "-g",
            "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in (os.path.join(ROOT, "long_context_sparse_amd", "csrc", "api.cpp"), os.path.join(SAN, "api_stubs.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *host, "-c", src, "-o", o], ROOT)
        objs.append(o)
    drv = str(tmp_path / "api_driver.o")
    _run([CLANG, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-c", os.path.join(SAN, "api_driver.cpp"), "-o", drv], ROOT)
    exe = str(tmp_path / "api_driver")
    _run([CLANG, "-fsanitize=address,undefined", *objs, drv, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe], ROOT)
    r = _run([exe], ROOT)
    assert "api driver clean" in r.stdout
