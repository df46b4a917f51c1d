"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (argument validation, size arithmetic, pass
planning: csrc/msa_api.hip) is compiled with host-only sanitizers and linked,
with the library's other objects, into tests/sanitize/abi_host_check.cpp, a
driver that calls every entry point with rejected arguments and every size
query over a sweep of shapes up to the limits.  No call reaches the GPU, so
this runs without one.  Device code is built as usual (sanitizers apply to
the host pass only).
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_abi_host_under_asan_and_ubsan():
    from block_sparse_long_index_amd import build as B
    objs = sorted(glob.glob(os.path.join(B.BUILD_DIR, "*.o")))
    if not any(o.endswith("msa_api.o") for o in objs):
        B.build_library(verbose=False)
        objs = sorted(glob.glob(os.path.join(B.BUILD_DIR, "*.o")))
    out = os.path.join(B.BUILD_DIR, "sanitize")
    os.makedirs(out, exist_ok=True)
    san_flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(out, "msa_api_san.o")
    cmd = [HIPCC, *B.FLAGS, "-O1", "-g", *san_flags, "-c", os.path.join(B.CSRC, "msa_api.hip"),
           "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    drv_obj = os.path.join(out, "abi_host_check.o")
    # the driver passes out-of-range enum values on purpose, as a C caller may (loading
    # them is undefined in C++ only): its own enum loads are not checked, the library's are
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize=enum",
           "-fno-sanitize-recover=all", "-I", B.INCLUDE, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"),
           "-o", drv_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(out, "abi_host_check")
    others = [o for o in objs if not o.endswith("msa_api.o")]
    cmd = [CLANG, "-fsanitize=address,undefined", "--hip-link", "-o", exe, drv_obj, api_obj, *others,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi host checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
