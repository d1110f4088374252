"""Build step for the CPU oracle: gcc, IEEE double, OpenMP.  Test infrastructure."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "dsa_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    # -ffp-contract=off keeps every multiply and add separately rounded, as written.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
