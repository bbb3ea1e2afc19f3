"""The C ABI from C++ alone (GPU required).  tests/c_abi/step_check.cpp, built by
__graft_entry__.build(), runs a layer's pipelined steps through include/asp.h
with hipMalloc'd buffers on one stream, on two streams with a context, and on
two streams with a context each in two host threads at once, and checks that
every step's output, selection and query ring agree bit for bit."""
import os
import subprocess

import pytest

from asp_testutil import require_gpu

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(__file__), "c_abi", "step_check")


def test_c_abi_pipelined_steps_agree_across_stream_modes():
    require_gpu()
    assert os.path.exists(BIN), "tests/c_abi/step_check is not built; run __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c-abi step check: ok" in r.stdout
    assert r.stdout.count("one stream and two streams agree; two threads with a context each agree") == 7


def test_c_abi_page_baseline():
    # tests/c_abi/page_check.cpp: one-token pages against the token-level
    # selection (bit for bit on small-integer inputs), and well-formed page
    # token lists with pages of 16.
    require_gpu()
    page_bin = os.path.join(os.path.dirname(__file__), "c_abi", "page_check")
    assert os.path.exists(page_bin), "tests/c_abi/page_check is not built; run __graft_entry__.build()"
    r = subprocess.run([page_bin], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "one-token pages and the token selection agree" in r.stdout
    assert "page token lists well-formed" in r.stdout
    assert "c-abi page check: ok" in r.stdout
