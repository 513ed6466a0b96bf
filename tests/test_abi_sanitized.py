"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp -- every entry point's argument checks, the work plan, the workspace
layout -- is compiled with the host-side sanitizers (the device code is not
instrumented: -Xarch_host applies the flags to the host pass only) and linked
with the other translation units into a separate library.  Against it run
the C program tests/c_abi_consumer.c (built with the same sanitizers) and the
ctypes ABI checks of tests/test_abi.py (with the sanitizer runtime
preloaded).  Every call there fails validation before any launch, so no GPU
is needed; a sanitizer report fails the test.
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_fp8_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _asan_runtime()):
        pytest.skip("hipcc, clang or the clang sanitizer runtime is not installed")
    d = tmp_path_factory.mktemp("sanitized")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = str(d / (src + ".o"))
        extra = (SAN + ["-x", "hip"]) if src == "api.cpp" else []
        subprocess.run([HIPCC, *flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        return obj

    srcs = ["api.cpp", "quant_append.hip", "decode_attn.hip", "page_pool.hip", "absmax.hip", "int4_gemv.hip"]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(d / "libfp8kv_sanitized.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-shared-libasan", *objs, "-o", lib],
                   check=True, capture_output=True)
    exe = str(d / "c_abi_consumer_sanitized")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-shared-libasan", "-I", INCLUDE, os.path.join(ROOT, "tests", "c_abi_consumer.c"), "-o", exe,
                    str(lib), f"-Wl,-rpath,{d}", "-lm"], check=True, capture_output=True)
    rt = _asan_runtime()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24",
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    return dict(lib=lib, exe=exe, runtime=rt, env=env)


def test_library_is_instrumented(sanitized):
    out = subprocess.run(["nm", "-D", sanitized["lib"]], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_" in out


def test_c_consumer_under_sanitizers(sanitized):
    res = subprocess.run([sanitized["exe"]], capture_output=True, text=True, env=sanitized["env"], timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "passed" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr


def test_ctypes_abi_checks_under_sanitizers(sanitized):
    env = dict(sanitized["env"], LD_PRELOAD=sanitized["runtime"], FP8KV_TEST_LIB=sanitized["lib"])
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                          "-p", "no:cacheprovider", "-k", "not c_program"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
