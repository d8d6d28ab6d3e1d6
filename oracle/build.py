"""Compile the CPU oracle (plain C, gcc) into oracle/libkda_oracle.so.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")

# No fast-math and no contraction: every double operation rounds as written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(out: str = LIB, src: str = SRC, extra=()) -> str:
    """Build the oracle library; return its path. Always recompiles."""
    tmp = f"{out}.tmp{os.getpid()}"  # per process: concurrent builds never share a file
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
