"""Build the CPU oracle library (liboracle.so) with gcc.

Test infrastructure: the oracle checks the HIP library and is never part of
its product path.  -ffp-contract=off and no -ffast-math keep every FP32
multiply and add a separate IEEE operation in the written order.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-std=c11", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile moe_oracle.c into liboracle.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
