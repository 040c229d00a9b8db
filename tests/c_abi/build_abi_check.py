"""Compile tests/c_abi/abi_check.c, a plain C consumer of libkda.so (test
infrastructure: it links the fp64 oracle's C source to check the results).

gcc builds it against include/kda.h and ROCm's HIP runtime headers as C99,
which also shows that the public header is valid C.  The binary finds
libkda.so and libamdhip64.so through its run path, relative to its own
location, so the tree can move.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
BIN = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out=BIN):
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-fopenmp", "-D__HIP_PLATFORM_AMD__",
            "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
            "-o", out, SRC, os.path.join(ROOT, "oracle", "kda_oracle.c"),
            "-L" + os.path.join(ROOT, "gated_delta_rule_25_amd"), "-lkda",
            "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_25_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(out=BIN):
    """Compile the consumer; raises CalledProcessError with gcc's output on failure."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(command(tmp), check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
