"""Build the CPU oracle library (test infrastructure only).

    python -m oracle.build

Compiles ring_oracle.c with gcc into oracle/libring_oracle.so.  The flags keep
every floating-point operation a single IEEE operation: no contraction into
FMA and no fast-math, so binary32 results are reproducible bit for bit.
"""
from __future__ import annotations

import os
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "ring_oracle.c"
LIB = HERE / "libring_oracle.so"

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> pathlib.Path:
    """Compile the oracle; always rebuilds.  Returns the library path."""
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", *CFLAGS, str(SRC), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
