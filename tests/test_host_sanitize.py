"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU needed).

kda_api.hip is compiled with both sanitizers on its host side only (each
-fsanitize after -Xarch_host; the device code is untouched), linked with
stub launch functions that abort and with the plain C program
tests/c_abi/host_sanitize.c, which drives every entry point through calls
that fail argument validation, plus the workspace queries and status
strings.  The test passes when the program exits 0 and neither sanitizer
reports anything.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CABI = os.path.join(ROOT, "tests", "c_abi")
INC = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "gated_delta_rule_25_amd", "csrc")]
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def _host_san():
    # every -fsanitize flag directly after -Xarch_host: host code only
    out = []
    for f in SAN:
        out += ["-Xarch_host", f]
    return out


@pytest.mark.skipif(not all(os.path.exists(x) for x in (HIPCC, CLANG, CLANGXX)), reason="ROCm toolchain missing")
def test_host_code_under_asan_and_ubsan(tmp_path):
    api = str(tmp_path / "api.o")
    stubs = str(tmp_path / "stubs.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "host_sanitize")
    base = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops"]
    steps = [
        [HIPCC] + base + _host_san() + INC + ["-c", os.path.join(ROOT, "gated_delta_rule_25_amd", "csrc", "kda_api.hip"),
                                              "-o", api],
        [CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + SAN + INC +
        ["-c", os.path.join(CABI, "launch_stubs.cpp"), "-o", stubs],
        [CLANG, "-O1", "-g", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + SAN +
        INC + ["-c", os.path.join(CABI, "host_sanitize.c"), "-o", drv],
        [CLANGXX] + SAN + [drv, api, stubs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, "build step failed:\n" + " ".join(cmd) + "\n" + r.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host sanitizer checks passed" in out
