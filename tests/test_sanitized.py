"""The CPU suite again, against host builds instrumented with AddressSanitizer
and UndefinedBehaviorSanitizer: libqsa's host code (argument checks,
workspace carving, the slot pool, the launch sequence; the device code is the
same) and the C oracle, both built with clang and sharing clang's ASan
runtime, which is preloaded into a fresh interpreter. Any report fails the
run (halt_on_error, no recovery from UBSan checks). The builds come from
__graft_entry__.build(); without them the test is skipped with that reason.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "kv_cache_selection_amd", "_build_san", "libqsa.so")
SAN_ORACLE = os.path.join(ROOT, "oracle", "_build", "libqsa_oracle_san.so")
ASAN_RT = "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    rts = sorted(glob.glob(ASAN_RT))
    if not (os.path.exists(SAN_LIB) and os.path.exists(SAN_ORACLE) and rts):
        pytest.skip("sanitized host builds not present (run __graft_entry__.build())")
    log = str(tmp_path / "san")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rts[-1],
        # the interpreter and torch are not instrumented: their leaks and
        # duplicate globals are not this library's
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:halt_on_error=1:log_path=" + log,
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:log_path=" + log,
        "QSA_LIBRARY": SAN_LIB,
        "QSA_ORACLE_SANITIZED": "1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-k", "not cpu_suite_under_asan", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert not reports, reports[:4000]
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout
