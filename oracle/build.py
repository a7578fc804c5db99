"""Compile the C oracle into oracle/libgpex_oracle.so with gcc (no GPU code involved).

TEST INFRASTRUCTURE ONLY: the oracle is loaded by tests, the smoke check and the CPU-baseline
leg of the benchmark, never by the HIP library or its Python binding."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpex_oracle.c")
LIB = os.path.join(HERE, "libgpex_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
