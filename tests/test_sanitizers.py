"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle's C sources built with gcc -fsanitize=address,undefined, driving the
  oracle pin suites (the planted-mistake tests are left out: they build
  deliberately broken copies of the oracle).
* The library's host code (argument checks, sizes, the host planner, the block
  pool; device code is unaffected: every sanitizer flag is host-only) built with
  hipcc and clang's sanitizers, driving the host ABI and block-pool tests.

Each suite runs in a child process with the matching sanitizer runtime
preloaded; a report fails the child (UBSan halts on the first error). A planted
out-of-bounds read first shows that the harness does report one.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip("gcc sanitizer runtime %s not found" % name)
        libs.append(p)
    return ":".join(libs)


def _clang_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang ASan runtime not found")
    return hits[-1]


def _run(cmd, preload, extra_env, timeout=900):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    return subprocess.run(cmd, capture_output=True, text=True, cwd=str(ROOT), env=env, timeout=timeout)


def _assert_clean(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_the_harness_reports_a_planted_out_of_bounds_read(tmp_path):
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint oob(int n) { int* a = malloc(4 * n); int v = a[n]; free(a); return v; }\n")
    so = tmp_path / "liboob.so"
    subprocess.run(["gcc", "-O0", "-g", "-fsanitize=address", "-fPIC", "-shared", str(src), "-o", str(so)], check=True)
    r = _run([sys.executable, "-c", "import ctypes; ctypes.CDLL(%r).oob(8)" % str(so)], _gcc_runtime(), {})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    so = tmp_path / "liboracle_san.so"
    srcs = [str(ROOT / "oracle" / f) for f in ("mla_oracle.c", "mla_oracle_sparse.c", "mla_oracle_fp8.c")]
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-std=c11", "-fPIC", "-shared", "-pthread", *srcs,
                    "-o", str(so), "-lm"], check=True)
    r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
              "-k", "not planted", "tests/test_oracle_pins.py", "tests/test_oracle_sparse.py",
              "tests/test_oracle_fp8.py", "tests/test_oracle_append.py"],
             _gcc_runtime(), {"MLA_ORACLE_LIB": str(so)})
    _assert_clean(r)
    assert " passed" in r.stdout


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    from mla_paged_latent_amd import build
    so = tmp_path / "libmla_san.so"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                "-Xarch_host", "-g"]
    build.build(out=so, extra_flags=host_san, objdir=tmp_path / "obj")
    r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
              "tests/test_host_abi.py", "tests/test_block_pool.py"],
             _clang_runtime(), {"MLA_LIB": str(so)})
    _assert_clean(r)
    assert " passed" in r.stdout
