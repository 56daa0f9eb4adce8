"""Build tests/probes/libcvtprobe.so (test-only) with the library's own hipcc flags."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libcvtprobe.so")


def build(verbose: bool = False) -> str:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from block_scaled_precision_mxfp8_amd import build as bsq_build

    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [bsq_build.hipcc(), *bsq_build.HIPCC_FLAGS, "-shared", "-x", "hip",
           os.path.join(HERE, "cvt_probe.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
