"""Compile the CPU oracle (plain C, double precision) into a shared library.

Test infrastructure: the oracle is what the GPU library is checked against.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every f32/double operation rounds
# once (x86-64 SSE arithmetic), as the definitions are written.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY, quiet: bool = False) -> str:
    """Compile `source` with gcc into `output` and return its path."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, source, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{res.stderr}")
    if res.stderr and not quiet:
        sys.stderr.write(res.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
