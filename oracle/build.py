"""Build the CPU oracle (``oracle/liboracle.so``) with gcc.

Test infrastructure only; see ``oracle/__init__.py``.  Flags: no fast-math
and no floating-point contraction, so the C compiler evaluates the k-sum
exactly as written; OpenMP only splits independent output entries.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
