"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU-side
code (CPU only; no GPU code runs with a sanitizer).

* The oracle (plain C) built with gcc -fsanitize=address,undefined runs the
  oracle pins (tests/test_oracle.py) through SFFN_ORACLE_SO.
* The library built with hipcc, host side only sanitized (-Xarch_host), runs
  the C-ABI validation tests (tests/test_abi.py and the CPU part of
  tests/test_zz_no_alloc.py) through SFFN_LIBRARY: every argument check,
  workspace size and handle path of abi.cpp and the entry points.
Any sanitizer report fails the run (halt_on_error)."""
import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from activation_sparse_gated_gate_amd import _build  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_pytest(args, env_extra):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", **SAN_ENV, **env_extra)
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", *args], cwd=ROOT,
                       env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    out = p.stdout.decode(errors="replace")
    assert p.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "oracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=undefined", "-Wno-unknown-pragmas",
                               os.path.join(ROOT, "oracle", "sffn_oracle.c"), "-o", so, "-lm"])
        asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
        _run_pytest([os.path.join(ROOT, "tests", "test_oracle.py")], {"SFFN_ORACLE_SO": so, "LD_PRELOAD": asan})


def test_library_host_code_under_asan_ubsan():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang ASan runtime")
    with tempfile.TemporaryDirectory() as td:
        san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-shared-libsan", "-Xarch_host", "-fno-sanitize-recover=undefined"]
        def compile_one(src):
            obj = os.path.join(td, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            subprocess.check_call([_build.HIPCC, *_build.COMMON, *_build.DEVICE_FLAGS, *san, *lang, "-c",
                                   os.path.join(_build.CSRC, src), "-o", obj],
                                  stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            objs = list(ex.map(compile_one, _build.SOURCES))
        so = os.path.join(td, "libsffn_san.so")
        subprocess.check_call([_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC",
                               "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libsan",
                               *objs, "-o", so])
        _run_pytest([os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_zz_no_alloc.py"),
                     "-m", "not gpu"], {"SFFN_LIBRARY": so, "LD_PRELOAD": rt[-1]})
