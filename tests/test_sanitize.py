"""Argument validation of every C entry point, from plain C, with the C ABI's
host code under AddressSanitizer and UndefinedBehaviorSanitizer
(tests/c_client/abi_validate.c, built twice by __graft_entry__.build()).

Every call passes an invalid argument through fake device pointers and must
return its documented error before launching anything; the sanitized build
also fails on an out-of-bounds access, a use after free or undefined
behaviour (such as a signed overflow in the size arithmetic) on those paths.
Runs on hosts without a GPU (the program declines to run where one is
visible)."""

import os
import subprocess

import pytest

CDIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client")


@pytest.mark.parametrize("name", ["abi_validate", "abi_validate_asan"])
def test_argument_validation(name):
    exe = os.path.join(CDIR, name)
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is missing: run __graft_entry__.build()")
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120, env=env)
    print(res.stdout[-3000:], flush=True)
    assert res.returncode == 0, res.stdout[-3000:]
    assert "validation checks passed" in res.stdout or "skipped" in res.stdout
    assert "runtime error" not in res.stdout and "AddressSanitizer" not in res.stdout
