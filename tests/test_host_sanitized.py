"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

fa_api.cpp is compiled by g++ with -fsanitize=address,undefined together with
fa_host_stubs.cpp (launchers that only report an error) into a host-only
library, and tests/test_abi.py runs against it in a subprocess with the ASan
runtime preloaded.  Every argument check, workspace size and status path of
test_abi then runs under the sanitizers; any report fails the run.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from causal_attention_fa_amd.build import build_host_sanitized
    lib = build_host_sanitized(str(tmp_path))
    asan = subprocess.check_output(["g++", "-print-file-name=libasan.so"], text=True).strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); import causal_attention_fa_amd as fa; "
            f"fa.library_path = {lib!r}; import pytest; "
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
