"""The C ABI's validation and sizing paths under AddressSanitizer and
UndefinedBehaviorSanitizer (host code): tests/helpers/abi_asan_check, built
from the library's sources and tests/helpers/abi_asan_check.cpp by
sub_byte_mixed_amd/build.py (build_asan_check, part of __graft_entry__.build),
calls every entry point with rejected arguments and every sizing helper over
a sweep of shapes; none of these calls reaches the GPU."""
import json
import os
import subprocess

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "helpers", "abi_asan_check")


def test_validation_and_sizing_clean_under_asan_and_ubsan():
    if not os.path.exists(BIN):
        from sub_byte_mixed_amd import build
        build.build_asan_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120, env=env)
    assert "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert out["failures"] == 0 and out["sized"] > 0
