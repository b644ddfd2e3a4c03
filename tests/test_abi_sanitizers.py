"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The library's sources are compiled with the sanitizers on the
host side only (device code as usual) and linked into
tests/abi_sanitize_driver.cpp, which drives argument validation, zero-sized
calls, workspace and plan queries and per-thread error messages over extreme
sizes, strides and leading dimensions (products that overflow int64
included).  Any sanitizer report, or a wrong status, fails the test.  Needs
no GPU; on a host that has one the driver declines to run and the test is
skipped."""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# Sanitizers on the host pass of each HIP compile (-Xarch_host before every
# sanitizer flag); the device code is built as usual and not instrumented.
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined").split()
LIB_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-fno-omit-frame-pointer", *HOST_SANITIZE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", INCLUDE, "-I", CSRC]
# The driver and the link step are host C++ only.
HOST_ONLY_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not installed")
    sources = ["quant.hip", "gemm.hip", "api.cpp"]
    cmds = [[HIPCC, *LIB_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, s),
             "-o", str(tmp_path / (s + ".o"))] for s in sources]
    cmds.append([CLANGXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
                 *HOST_ONLY_SANITIZE, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                 "-I", INCLUDE, "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"),
                 "-o", str(tmp_path / "driver.o")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, cmds))
    exe = tmp_path / "abi_sanitize_driver"
    _run([CLANGXX, *HOST_ONLY_SANITIZE, str(tmp_path / "driver.o"),
          *[str(tmp_path / (s + ".o")) for s in sources],
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
          "-lpthread", "-o", str(exe)])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=1:strict_string_checks=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    report = r.stdout + r.stderr
    assert "Sanitizer" not in report and "runtime error" not in report, report[-6000:]
    assert r.returncode == 0, report[-6000:]
    assert "0 failures" in r.stdout, report[-6000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
