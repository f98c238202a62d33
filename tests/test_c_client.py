"""The library from a plain C program (tests/c_client/abi_client.c, built by
__graft_entry__.build()): no Python and no torch between the caller and the
C ABI.  On the CPU only its argument checks run; on a GPU it also checks the
one-key and uniform-attention closed forms and the bf16 path against the fp32
path."""

import os
import subprocess

import pytest

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "abi_client")


def _run(*args):
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client/abi_client is missing: run __graft_entry__.build()")
    res = subprocess.run([CLIENT, *args], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=120)
    print(res.stdout, flush=True)
    return res


def test_c_client_argument_errors():
    res = _run("--no-gpu")
    assert res.returncode == 0 and "argument checks passed" in res.stdout


@pytest.mark.gpu
def test_c_client_on_gpu():
    res = _run()
    assert res.returncode == 0 and "all checks passed" in res.stdout
