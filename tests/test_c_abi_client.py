"""The C ABI from C: tests/c_abi_client.c includes include/fp8bw.h, links
libfp8bw.so and runs host-only calls (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from blockwise_scaled_fp8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_builds_links_and_runs(tmp_path):
    lib = _lib.lib_path()
    if not os.path.exists(lib):
        pytest.fail("libfp8bw.so is not built (run __graft_entry__.build())")
    cc = shutil.which("gcc") or shutil.which("cc")
    assert cc, "no C compiler"
    exe = tmp_path / "client"
    libdir = os.path.dirname(lib)
    subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_client.c"), "-L", libdir, "-l:libfp8bw.so",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi client ok" in r.stdout
