"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

fa_api.cpp (argument checks, workspace sizes, dispatch) is compiled with g++ and the sanitizers, linked with
the library's kernel objects (built as usual, not instrumented) into a separate library, and every case of
tests/test_abi.py runs against it in a child process with the sanitizer runtimes preloaded. Any invalid
memory access or undefined behaviour on those paths ends the child with a sanitizer report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tiled_online_softmax_fa_amd")
BUILD = os.path.join(PKG, "_build")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _runtime(gxx, name):
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_cases_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    kernels = sorted(p for p in glob.glob(os.path.join(BUILD, "*.o")) if not p.endswith("fa_api.o"))
    if len(kernels) < 4:
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    asan, ubsan = _runtime(gxx, "libasan.so"), _runtime(gxx, "libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not found")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    obj = str(tmp_path / "fa_api_asan.o")
    lib = str(tmp_path / "libfa_asan.so")
    cc = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-c",
          os.path.join(PKG, "csrc", "fa_api.cpp"), "-o", obj]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    ld = [gxx, "-shared", *SAN, obj, *kernels, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", lib]
    r = subprocess.run(ld, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{asan}:{ubsan}", FA_ABI_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x", "-s",
                        "-p", "no:cacheprovider"], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
