"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  * the fp64 oracle (oracle/msa_oracle.c), built with gcc
    -fsanitize=address,undefined, runs the oracle's pins and the caller-table
    pins (tests/test_oracle.py, tests/test_tables.py, without the planted-
    mistake builds) in a child process with gcc's sanitizer runtimes preloaded;
  * the library's host code (csrc/msa.cpp: validation, workspace planning,
    dispatch; csrc/noalloc.hip's host side), compiled by hipcc with the
    sanitizers on the host pass only (-Xarch_host before each -fsanitize=) and
    linked with the kernel objects of the ordinary build, runs the ABI tests
    (tests/test_abi.py: every validation and refusal path, workspace sizes)
    with clang's ASan runtime preloaded.
Any report fails the child (UBSan is made fatal; leak checking is off, the
interpreter itself keeps memory until exit).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_bk_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _gcc_rt(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_rt():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _child(code, preload, timeout=900):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


CHECK_LOADED = """
import ctypes
def _loaded(path):
    assert path in open('/proc/self/maps').read(), path + ' is not the loaded copy'
    assert hasattr(ctypes.CDLL(None), '__asan_report_load8'), 'the ASan runtime is not in the process'
"""


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_rt("libasan.so"), _gcc_rt("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "libmsa_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-o", lib, os.path.join(ROOT, "oracle", "msa_oracle.c"), "-lm"], check=True)
    code = CHECK_LOADED + f"""
import sys
from oracle import oracle as O
O._default = O.Oracle({lib!r})
_loaded({lib!r})
import pytest
sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-k', 'not planted', '-p', 'no:cacheprovider',
                      'tests/test_oracle.py', 'tests/test_tables.py']))
"""
    out = _child(code, f"{asan}:{ubsan}")
    assert " passed" in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    rt = _clang_asan_rt()
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's ASan runtime is not installed")
    kernels = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
               if os.path.basename(s) != "noalloc.hip"]
    if not all(os.path.exists(o) for o in kernels):
        from block_sparse_long_bk_amd import build as hip_build
        hip_build.build()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host_objs = []
    for src in ("msa.cpp", "noalloc.hip"):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([HIPCC, *flags, *SAN_HOST, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        host_objs.append(obj)
    lib = str(tmp_path / "libmsa_san.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, *kernels, *host_objs],
                   check=True, capture_output=True)
    code = CHECK_LOADED + f"""
import sys
from block_sparse_long_bk_amd import api
api.LIB_PATH = {lib!r}
api.lib()
_loaded({lib!r})
import pytest
sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', 'tests/test_abi.py']))
"""
    out = _child(code, rt)
    assert " passed" in out
