"""The C ABI used from plain C: tests/c_abi/consumer.c quantizes and dequantizes through
include/bsq.h with the HIP runtime's C API only, and compares every byte with the CPU
oracle; it also checks that argument errors return at once and leave outputs untouched.
The program is built by __graft_entry__.build() (tests/c_abi/build_consumer.py)."""
import os
import subprocess

import pytest

from gpu_helpers import log

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "consumer")


@pytest.mark.parametrize("M,K", [(256, 2048), (96, 160), (4128, 736)])
def test_plain_c_consumer_matches_oracle(M, K):
    assert os.path.exists(EXE), "tests/c_abi/consumer is not built; run __graft_entry__.build()"
    log("c consumer %dx%d" % (M, K))
    r = subprocess.run([EXE, str(M), str(K)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all equal" in r.stdout
