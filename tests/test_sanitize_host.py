"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only).

gqa_api.cpp -- argument checks, the split planner, workspace sizing, the
launch set-up -- is built with the sanitizers on its host code, and linked
with stand-in launchers (tests/c/launch_stubs.cpp) instead of the GPU
kernels: each stand-in checks on the host that the launch it is handed fits
what the kernel assumes, and enqueues nothing.  Three drivers run against
that build: a seeded sweep of edge-value parameters (tests/c/abi_sweep.c),
the C99 header check (tests/c/abi_host.c), and the Python ABI and binding
tests with the sanitizer runtime preloaded.  Any out-of-bounds access,
signed overflow, misaligned load or unfit launch fails the test.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_kv_cache_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CDIR = os.path.join(ROOT, "tests", "c")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and ASAN_RT),
                                reason="needs ROCm's hipcc, clang and the sanitizer runtime")


@pytest.fixture(scope="module")
def hostcheck(tmp_path_factory):
    d = tmp_path_factory.mktemp("hostcheck")
    lib = str(d / "libgqa_hostcheck.so")
    # Sanitizers on the host code only: each -fsanitize= follows -Xarch_host.
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-fno-omit-frame-pointer",
           f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "gqa_api.cpp"),
           os.path.join(CDIR, "launch_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return d, lib


def _c_driver(d, lib, src, name):
    exe = str(d / name)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd = [CLANG, "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *san, f"-I{INCLUDE}",
           os.path.join(CDIR, src), lib, f"-Wl,-rpath,{d}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_parameter_sweep(hostcheck):
    d, lib = hostcheck
    exe = _c_driver(d, lib, "abi_sweep.c", "abi_sweep")
    for seed in (1, 2, 3):
        r = subprocess.run([exe, "300000", str(seed)], capture_output=True, text=True, timeout=600, env=ENV)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert "0 failures" in r.stdout


def test_c_header_program(hostcheck):
    d, lib = hostcheck
    exe = _c_driver(d, lib, "abi_host.c", "abi_host")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


def test_python_abi_tests(hostcheck):
    d, lib = hostcheck
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import gqa_kv_cache_amd as G\n"
            "G.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r, %r]))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py"),
               os.path.join(ROOT, "tests", "test_binding_checks.py")))
    env = dict(ENV, LD_PRELOAD=ASAN_RT[-1])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
