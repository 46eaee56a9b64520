"""The public headers from C: a C99 program includes include/*.h, links
against the built libgqa_decode.so and drives the host side of the ABI
(planning, workspace sizes, status strings, argument checks) with no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "gqa_kv_cache_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_and_link_from_c(tmp_path):
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), os.path.join(LIB_DIR, "libgqa_decode.so"),
           "-Wl,-rpath," + LIB_DIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
