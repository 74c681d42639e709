"""Builds the C-ABI consumer program (test infrastructure) with the host C
compiler: the library's headers compiled as C99, the program linked against
the in-tree libce.so and the HIP runtime, nothing else."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "softmax_cross_entropy_fwd_amd")
SRC = os.path.join(HERE, "ce_consumer.c")
EXE = os.path.join(HERE, "ce_consumer")
ROCM = "/opt/rocm"


def command(out):
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
            "-o", out, "-L", PKG, "-lce", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            # the library next to the program's tree wherever the tree is copied,
            # then this tree's absolute path, then ROCm's
            "-Wl,-rpath,$ORIGIN/../../softmax_cross_entropy_fwd_amd", "-Wl,-rpath," + PKG,
            "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(out=EXE):
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(command(tmp), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
