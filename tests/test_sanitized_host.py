"""CPU: the host planner and the C ABI's host paths under the address and
undefined-behaviour sanitizers.

The library is rebuilt with both sanitizers on its host code (device code as
usual; tree_structured_shared_amd.build, sanitize=True) and then
* tests/native/abi_driver.c, built with the same sanitizers and leak
  checking on, plans, exports and grows 300 random trees host-only, walks
  every host allocation step of ta_plan_opts.fail_alloc_after (TA_ENOMEM,
  no leak, the plan usable after a failed extend's host step) and every
  documented error code;
* the bit-exact planner tests (1,000 random trees against the Python
  re-derivation), the decode-loop extend tests, the ABI error tests and the
  planner property tests run in a Python process that preloads the sanitizer
  runtime and loads the sanitized library (TREE_ATTN_LIB).
Any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

from tree_structured_shared_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:")


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    rt = B.asan_runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("no sanitizer runtime in this toolchain")
    out = str(tmp_path_factory.mktemp("san") / "libtree_attn_san.so")
    B.build(out=out, sanitize=True)
    return out, rt


def _clean(res):
    text = res.stdout + res.stderr
    assert not any(r in text for r in REPORTS), text[-4000:]
    assert res.returncode == 0, text[-4000:]


def test_c_driver_under_sanitizers(san_lib, tmp_path):
    lib, rt = san_lib
    exe = str(tmp_path / "abi_driver")
    cc = subprocess.run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libasan",
                         "-g", "-O1", f"-I{os.path.join(ROOT, 'include')}",
                         os.path.join(ROOT, "tests", "native", "abi_driver.c"), lib,
                         f"-Wl,-rpath,{os.path.dirname(lib)}", f"-Wl,-rpath,{os.path.dirname(rt)}", "-o", exe],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    _clean(res)
    assert res.stdout.startswith("ok "), res.stdout


def test_planner_suites_under_sanitizers(san_lib):
    lib, rt = san_lib
    env = dict(os.environ, LD_PRELOAD=rt, TREE_ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c",
                            "from tree_structured_shared_amd import _capi; _capi.lib(); "
                            "print(open('/proc/self/maps').read().count('libtree_attn_san.so') > 0)"],
                           capture_output=True, text=True, env=env, timeout=300, cwd=ROOT)
    assert probe.stdout.strip().endswith("True"), probe.stdout + probe.stderr  # the sanitized build is the one loaded
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_planner_capi.py"),
                          os.path.join(ROOT, "tests", "test_plan_extend.py"),
                          os.path.join(ROOT, "tests", "test_planner_props.py")],
                         capture_output=True, text=True, env=env, timeout=1200, cwd=ROOT)
    _clean(res)
    assert " passed" in res.stdout, res.stdout[-2000:]
