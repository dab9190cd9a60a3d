"""The host code under the address and undefined-behaviour sanitizers (CPU only): the C ABI's
host side (argument checks, plans, workspace layouts, dispatch; the device launchers replaced by
stand-ins that fail) and the float64 oracle, each built into a small driver program with clang
and run.  A memory error, a leak in the oracle or undefined behaviour stops the program with a
report; the drivers also check every returned status and a few values."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "fft_long_convolution_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _tool(name):
    p = os.path.join(LLVM, name)
    if not os.path.exists(p):
        pytest.skip(f"{p} not found")
    return p


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-6000:]
    return r


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_sanitizers(outdir):
    cc = _tool("clang")
    exe = os.path.join(outdir, "oracle_san")
    _run([cc, *SAN, "-std=c11", "-pthread", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(HERE, "oracle_main.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert "ORACLE_SANITIZED_OK" in r.stdout


def test_abi_host_code_under_sanitizers(outdir):
    cxx = _tool("clang++")
    rocm = "/opt/rocm"
    if not os.path.exists(os.path.join(rocm, "lib", "libamdhip64.so")):
        pytest.skip("HIP runtime library not found")
    exe = os.path.join(outdir, "abi_san")
    srcs = [os.path.join(CSRC, "lconv_api.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(HERE, "stubs.cpp"),
            os.path.join(HERE, "abi_main.cpp")]
    _run([cxx, *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-result", "-Wno-unused-value", *srcs,
          "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe])
    # the HIP runtime's own allocations are not this code's: leak checking off for this program
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = _run([exe], env=env)
    assert "ABI_SANITIZED_OK" in r.stdout
