"""TEST INFRASTRUCTURE ONLY: compiles the CPU oracle (plain C, gcc, OpenMP).

No contraction of a*b+c into fma (-ffp-contract=off) and no fast-math, so the
fp32 evaluation order written in the source is the one executed.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = [os.path.join(HERE, "gs_oracle.c")]
DEPS = SRC + [os.path.join(HERE, "gs_oracle_body.h")]


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in DEPS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wno-unused-function", "-o", tmp] + SRC + ["-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
