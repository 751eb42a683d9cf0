"""Sanitizer runs on the CPU: the oracle under gcc's UndefinedBehaviorSanitizer and
AddressSanitizer, and the HIP library's host code (argument validation, launch
set-up; device code is not instrumented) under clang's UndefinedBehaviorSanitizer.

Each run builds the sanitized library beside the normal one (oracle.build(sanitize=...),
quantized_softmax_attention_amd.build.build_ubsan()), then runs a test subset in a
subprocess with that library swapped in (UBSan aborts on the first report:
-fno-sanitize-recover=all; ASan aborts on any error).  A positive control first
plants the kind of fault each mode must catch, so a run that reports nothing is
known to be live."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle
from quantized_softmax_attention_amd import build as lib_build
from quantized_softmax_attention_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["tests/test_oracle_attn.py", "tests/test_oracle_codec.py", "tests/test_oracle_quant.py",
                "tests/test_oracle_mx.py", "tests/test_oracle_norm_rope.py", "tests/test_golden_regression.py",
                "tests/test_pages_facts.py"]
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_binding_host.py"]


def _runtime(cc, name):
    path = subprocess.run([cc, "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


GCC_ASAN = _runtime("gcc", "libasan.so")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANG_UBSAN = _runtime(CLANG, "libclang_rt.ubsan_standalone-x86_64.so") if os.path.exists(CLANG) else None


def _run(tests, oracle_lib=None, sage_lib=None, preload=None, extra_env=None):
    code = textwrap.dedent("""
        import sys
        sys.path.insert(0, {root!r})
        import oracle
        from quantized_softmax_attention_amd import sage
        if {olib!r}:
            oracle._LIB = {olib!r}
        if {slib!r}:
            sage.LIB_PATH = {slib!r}
        import pytest
        sys.exit(pytest.main({args!r}))
        """).format(root=ROOT, olib=oracle_lib, slib=sage_lib,
                    args=["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *tests])
    env = dict(os.environ)
    if preload:
        env["LD_PRELOAD"] = preload
    env.update(extra_env or {})
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=900)


def _control(tmp_path, cc, flags, body, preload=None, extra_env=None):
    """A one-function shared library with a planted fault, called through ctypes under the runtime."""
    src = tmp_path / "fault.c"
    src.write_text(body)
    so = tmp_path / "libfault.so"
    subprocess.run([cc, "-O0", "-fPIC", "-shared", *flags, str(src), "-o", str(so)], check=True)
    code = "import ctypes, sys; L = ctypes.CDLL(%r); print(L.fault(int(sys.argv[1])))" % str(so)
    env = dict(os.environ)
    if preload:
        env["LD_PRELOAD"] = preload
    env.update(extra_env or {})
    return subprocess.run([sys.executable, "-c", code, "2147483647"], env=env, capture_output=True, text=True,
                          timeout=120)


OVERFLOW = "int fault(int x) { return x + 1; }\n"              # signed overflow for x = INT_MAX
HEAP = ("#include <stdlib.h>\nint fault(int x) { char *p = malloc(8); int r = p[8 + (x & 0)]; free(p);"
        " return r; }\n")                                      # reads one byte past an 8-byte block
ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0"}


def test_oracle_under_ubsan(tmp_path):
    ctl = _control(tmp_path, "gcc", oracle.SANITIZERS["ubsan"], OVERFLOW)
    assert ctl.returncode != 0 and "runtime error" in ctl.stderr, ctl.stderr[-500:]
    lib = oracle.build(sanitize="ubsan")
    r = _run(ORACLE_TESTS, oracle_lib=lib)
    assert r.returncode == 0 and "runtime error" not in r.stderr, (r.stdout[-2000:], r.stderr[-2000:])


@pytest.mark.skipif(GCC_ASAN is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_under_asan(tmp_path):
    ctl = _control(tmp_path, "gcc", oracle.SANITIZERS["asan"], HEAP, preload=GCC_ASAN, extra_env=ASAN_ENV)
    assert ctl.returncode != 0 and "heap-buffer-overflow" in ctl.stderr, ctl.stderr[-500:]
    lib = oracle.build(sanitize="asan")
    r = _run(ORACLE_TESTS, oracle_lib=lib, preload=GCC_ASAN, extra_env=ASAN_ENV)
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in r.stderr, (r.stdout[-2000:], r.stderr[-2000:])


@pytest.mark.skipif(CLANG_UBSAN is None or not os.path.exists(sage.LIB_PATH),
                    reason="clang's UBSan runtime or the HIP library is missing")
def test_library_host_code_under_ubsan(tmp_path):
    flags = [f for f in lib_build.UBSAN_FLAGS if f != "-Xarch_host"]
    ctl = _control(tmp_path, CLANG, flags, OVERFLOW, preload=CLANG_UBSAN)
    assert ctl.returncode != 0 and "runtime error" in ctl.stderr, ctl.stderr[-500:]
    lib = lib_build.build_ubsan()
    r = _run(HOST_TESTS, sage_lib=lib, preload=CLANG_UBSAN)
    assert r.returncode == 0 and "runtime error" not in r.stderr, (r.stdout[-2000:], r.stderr[-2000:])
