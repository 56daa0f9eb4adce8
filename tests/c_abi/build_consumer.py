"""Build tests/c_abi/consumer (test-only): a plain C program linked against libbsq.so,
the C oracle and the HIP runtime, with run paths relative to itself."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "consumer")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "consumer.c"), "-o", tmp,
           "-L", os.path.join(ROOT, "block_scaled_precision_mxfp8_amd"), "-lbsq",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../block_scaled_precision_mxfp8_amd:$ORIGIN/../../oracle:" + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
