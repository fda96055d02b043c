"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

Flags: no fast-math and no FP contraction, so every fp32 step of the quantizer is a single
IEEE-rounded operation and every fp64 sum is evaluated exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", os.path.join(HERE, "msa_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
