"""Sanitizer builds of the host-side code, no GPU needed.

- The CPU oracle (``oracle/moe_oracle.c``) built with AddressSanitizer and
  UndefinedBehaviorSanitizer (gcc), running its own pin tests
  (``tests/test_oracle.py``).
- The HIP library's host side (argument checks, workspace carving, every C
  entry point's validation) built with the same sanitizers on the host pass
  only (hipcc ``-Xarch_host``; device code is built as usual and never run
  here), running the C-ABI tests (``tests/test_abi.py``).

Each run is a child Python with the sanitizer runtime preloaded (the
interpreter itself is not instrumented) and recovery off, so any finding
aborts the child and fails the test.  The HIP build (about a minute) is
cached under ``_build/sanitize/`` by a digest of the sources.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(preload, code, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    return out


def _gcc_runtime():
    return ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                                   check=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))


@pytest.mark.parametrize("flag,call,report", [
    ("-fsanitize=address", "L.planted_oob(3); L.planted_oob(8)", "heap-buffer-overflow"),
    ("-fsanitize=undefined", "L.planted_add(5); L.planted_add(2147483647)", "signed integer overflow"),
])
def test_harness_catches_planted_bugs(tmp_path, flag, call, report):
    """The child set-up reports a heap overflow (AddressSanitizer) and a signed overflow
    (UndefinedBehaviorSanitizer) planted in a throwaway C file, and fails."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted_oob(int i) { int *a = malloc(8 * sizeof(int)); a[i] = 1; int r = a[0]; free(a); "
                   "return r; }\n"
                   "int planted_add(int x) { return x + 1; }\n")
    lib = str(tmp_path / "libplanted.so")
    subprocess.check_call(["gcc", "-O0", "-g", flag, "-fno-sanitize-recover=undefined", "-shared", "-fPIC",
                           str(src), "-o", lib])
    env = dict(os.environ, LD_PRELOAD=_gcc_runtime(), **SAN_ENV)
    code = f"import ctypes; L = ctypes.CDLL({lib!r}); {call}"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]


def _dynamic_symbols(path):
    return subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                           "-std=c11", os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"])
    syms = _dynamic_symbols(lib)
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the build is instrumented
    out = _child(_gcc_runtime(), f"""
import sys, pytest, oracle
oracle.use_library({lib!r})
sys.exit(pytest.main(['tests/test_oracle.py', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu']))
""")
    assert " passed" in out and "failed" not in out


def _san_hip_library():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                  + [os.path.join(ROOT, "include", "moe_q4.h")])
    digest = hashlib.sha256(b"".join(open(p, "rb").read() for p in srcs)).hexdigest()[:16]
    out_dir = os.path.join(ROOT, "_build", "sanitize", digest)
    lib = os.path.join(out_dir, "libmoe_q4_san.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(out_dir, exist_ok=True)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, "-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang",
                                       "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                                       "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-4000:]
    tmp = lib + ".tmp"
    subprocess.check_call([CLANG, "-shared", "-fsanitize=address,undefined", "-shared-libasan", *objs,
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp])
    os.replace(tmp, lib)
    return lib


@pytest.mark.timeout(900)
def test_host_abi_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    lib = _san_hip_library()
    syms = _dynamic_symbols(lib)
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "clang's ASan runtime not found"
    out = _child(rt[0], f"""
import sys, pytest
import quantized_moe_expert_amd._lib as L
L.LIB_PATH = {lib!r}
sys.exit(pytest.main(['tests/test_abi.py', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu']))
""")
    assert " passed" in out and "failed" not in out
