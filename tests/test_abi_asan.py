"""Host AddressSanitizer run of the C-ABI's argument validation (CPU only).

The host side of the entry points (api.cpp, profile.cpp) is rebuilt with
AddressSanitizer and linked with the ordinary kernel objects of the in-tree
build; the CPU ABI tests (test_abi_cpu.py) then run against that library in a
child process with the sanitizer runtime preloaded.  A sanitizer report of a
host memory error, or any failing ABI test, fails this test.  Device code is
not instrumented."""
import os
import subprocess
import sys

import pytest

from sparse_attention_17_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SOURCES = [s for s in build.SOURCES if s.endswith(".cpp")]
KERNEL_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _asan_runtime():
    for cc in ("/opt/rocm/llvm/bin/clang++", build.hipcc()):
        if not os.path.exists(cc):
            continue
        r = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                           capture_output=True, text=True)
        path = r.stdout.strip()
        if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
            return path
    return None


def test_abi_validation_under_host_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    kobjs = [os.path.join(build.OBJ, os.path.splitext(s)[0] + ".o") for s in KERNEL_SOURCES]
    if not all(os.path.exists(o) for o in kobjs):
        build.build()
    hipcc = build.hipcc()
    flags = [f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++20", "-fPIC",
             "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", build.CSRC]
    hobjs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        subprocess.run([hipcc, *flags, "-Xarch_host", "-fsanitize=address",
                        "-c", os.path.join(build.CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        hobjs.append(obj)
    lib = str(tmp_path / "libcsa_mi355x_asan.so")
    subprocess.run([hipcc, f"--offload-arch={build.ARCH}", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", *hobjs, *kobjs, "-o", lib],
                   check=True, capture_output=True)
    env = dict(os.environ, CSA_TEST_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
