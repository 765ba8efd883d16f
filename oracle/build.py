"""Build the oracle's shared library (plain C, gcc, no FMA contraction).

Test infrastructure: the oracle is only ever loaded by the tests, the smoke
check and the benchmark's CPU-baseline leg.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-fPIC", "-shared", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a modified copy of the oracle source (used by the tests that
    check the pins catch planted mistakes)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-w", "-fPIC",
                    "-shared", "-o", out_path, src, "-lm"], check=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
