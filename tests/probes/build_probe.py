"""Build the test-only probe libraries with the library's own hipcc flags:
tests/probes/libcvtprobe.so (conversion helpers over binary32 ranges, for the tests) and
tests/probes/libhbmprobe.so (byte-moving kernels without arithmetic, for
`bench.py --hbm-ceiling`)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libcvtprobe.so")
HBM_LIB = os.path.join(HERE, "libhbmprobe.so")


def _build_one(src: str, lib: str, verbose: bool) -> str:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from block_scaled_precision_mxfp8_amd import build as bsq_build

    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [bsq_build.hipcc(), *bsq_build.HIPCC_FLAGS, "-shared", "-x", "hip",
           os.path.join(HERE, src), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _build_one("hbm_probe.hip", HBM_LIB, verbose)
    return _build_one("cvt_probe.hip", LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
