"""Sanitizer builds on the host (no GPU needed): the CPU oracle under
AddressSanitizer and UndefinedBehaviorSanitizer over every entry point
(tests/sanitize_oracle.c), and the library's host code -- argument
validation and the host queries of every entry point -- built with the same
sanitizers for the host side only (tests/sanitize_abi.cpp).  Each run must
exit 0 with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    return report


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c99", "-g", "-O1", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), "-o", exe,
                    os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-lm"], check=True)
    assert "sanitized oracle run ok" in _run(exe)


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_library_host_code_under_asan_ubsan(tmp_path):
    obj, drv, exe = (str(tmp_path / n) for n in ("sv_abi.o", "drv.o", "abi_san"))
    csrc = os.path.join(ROOT, "draft_token_verification_11_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    # device code built as usual; the sanitizers apply to the host side only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-c", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san +
                   ["-I", inc, "-I", csrc, "-o", obj, os.path.join(csrc, "sv_abi.hip")],
                   check=True, capture_output=True)
    subprocess.run([CLANG, "-c", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", inc, "-o", drv,
                    os.path.join(ROOT, "tests", "sanitize_abi.cpp")], check=True)
    subprocess.run([CLANG, "-fsanitize=address,undefined", "-o", exe, obj, drv,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    assert "sanitized host validation ok" in _run(exe)
