"""The library's host code (the C ABI's argument validation, the launch
configuration and workspace sizing) under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU ABI and binding tests run again in a
child process against a build whose host pass is instrumented, with the ASan
runtime preloaded.  Any report aborts the child and fails this test."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT


def test_cpu_abi_tests_pass_under_asan_and_ubsan():
    B = pytest.importorskip("fp4_decode_gemv_amd.build")
    try:
        B.hipcc()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized(os.path.join(ROOT, "_build", "hostsan"))
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef, "the host code is not instrumented"
    code = (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]\n"
        "import fp4_decode_gemv_amd as F\n"
        f"F.LIB_PATH = {lib!r}\n"
        "assert F.lib()._name == F.LIB_PATH\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_host.py',"
        " 'tests/test_binding_host.py']))\n"
    )
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
