"""Build the CPU oracle (test infrastructure): ``python oracle/build.py``.

Compiles ``oracle.c`` with gcc into ``liboracle.so`` next to it.  ``-ffp-contract=off`` keeps
the compiler from fusing multiplies and adds on its own, so the only fused operations are the
explicit ``fmaf`` calls of the stated FP32 accumulation order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out=LIB, src=SRC, extra=()):
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
