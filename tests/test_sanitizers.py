"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (argument validation, workspace sizing, dispatch in
api.cpp) is rebuilt with host-only ASan/UBSan instrumentation and linked with
the library's other objects; the fp64 oracle is rebuilt with the same
sanitizers (single-threaded).  The ABI and oracle test files then run against
those builds in a child process with the sanitizer runtime preloaded; any
sanitizer report fails the test.  A planted out-of-bounds read in a throwaway
C file shows first that the instrumented toolchain does report such errors.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# Instrumentation of host code only: every sanitizer flag of a hipcc line is bound to the host pass.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def _env(extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **extra)
    return env


needs_toolchain = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _asan_runtime()),
                                     reason="ROCm clang with the ASan runtime is not installed")


@needs_toolchain
def test_sanitizer_reports_a_planted_error(tmp_path):
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { int* a = malloc(4 * sizeof(int)); "
                   "int x = a[c + 3]; free(a); return x & 0; }\n")
    exe = tmp_path / "oob"
    _run([CLANG, "-g", "-fsanitize=address", "-shared-libsan", str(src), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=_env({}))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


@needs_toolchain
def test_abi_and_oracle_tests_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    obj_dir = os.path.join(ROOT, "_build", "obj")
    csrc = os.path.join(ROOT, "sparse_attention_long_fwd_amd", "csrc")
    if not os.path.exists(os.path.join(obj_dir, "api.cpp.o")):
        sys.path.insert(0, ROOT)
        from sparse_attention_long_fwd_amd import build
        build.build()
    api_o = os.path.join(OUT, "api.o")
    _run([HIPCC] + HIP_FLAGS + HOST_SAN + ["-c", os.path.join(csrc, "api.cpp"), "-o", api_o])
    others = sorted(o for o in glob.glob(os.path.join(obj_dir, "*.o")) if not o.endswith("api.cpp.o"))
    lib = os.path.join(OUT, "libnsa_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SAN[:4] + ["-shared-libsan", "-o", lib, api_o] +
         others)
    nm = _run(["nm", "-D", lib]).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    olib = os.path.join(OUT, "libnsa_oracle_san.so")
    _run([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-fno-fast-math", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-shared-libsan", os.path.join(ROOT, "oracle", "nsa_oracle.c"), "-o",
          olib, "-lm"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle.py")],
                       capture_output=True, text=True, cwd=ROOT,
                       env=_env({"NSA_LIB_PATH": lib, "NSA_ORACLE_LIB_PATH": olib}))
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert not any(m in text for m in REPORTS), text[-4000:]
    assert " passed" in r.stdout
