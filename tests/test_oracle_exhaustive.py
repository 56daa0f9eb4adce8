"""The oracle's E4M3, E2M1 and BF16 encoders against independent bit-manipulation encoders
on every non-NaN binary32 input (2^32 - 2^24 + 2 values), in C with OpenMP
(tests/exhaustive/enc_sweep.c).  The oracle searches tables of the formats' values built
from their bit fields; the sweep's encoders round the binary32 significand directly.
Passages: page "Towards Blackwell-native 8-bit and 4-bit RL", section "Format background"
(E4M3 block scales and elements, E2M1 elements) and section "High-precision and
dequantized backward" (BF16 operands)."""
import os
import subprocess

import oracle
from host_env import child_env

HERE = os.path.dirname(os.path.abspath(__file__))


def test_encoders_agree_on_every_binary32_value(tmp_path):
    lib = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "liboracle.so")
    if not os.path.exists(lib):
        oracle.build()
    exe = os.path.join(str(tmp_path), "enc_sweep")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-Wall", "-Wextra", "-Werror", os.path.join(HERE, "exhaustive", "enc_sweep.c"),
                    "-L" + os.path.dirname(lib), "-l:" + os.path.basename(lib),
                    "-Wl,-rpath," + os.path.dirname(lib), "-o", exe], check=True)
    env = child_env()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" 0 mismatches") == 3
