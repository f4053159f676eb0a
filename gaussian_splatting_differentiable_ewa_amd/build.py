"""Builds the gfx950 HIP library ``libgs_hip.so`` in-tree with hipcc.

Flags:
  --offload-arch=gfx950            MI355X (CDNA4) code objects only
  -ffp-contract=fast-honor-pragmas contraction allowed except where a
                                   ``#pragma clang fp contract(off)`` pins the
                                   evaluation order (the decision path)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division and sqrt
  -munsafe-fp-atomics              hardware fp32 atomic add in the backward
  -target-feature -packed-fp32-ops no packed fp32 instructions
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgs_hip.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=fast-honor-pragmas", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source into one shared library (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra) + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out:
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
