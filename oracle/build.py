"""Compile the CPU oracle (plain C, gcc) into oracle/libecho_oracle.so.

Test infrastructure only.  -ffp-contract=off keeps every a*b+c unfused
(the oracle's only fused multiply-add is its explicit fmaf); -fno-fast-math
keeps IEEE semantics.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "echo_oracle.c")


def library_path() -> str:
    """Built library; ECHO_ORACLE_LIB may point at another build of the same source."""
    return os.environ.get("ECHO_ORACLE_LIB") or os.path.join(HERE, "libecho_oracle.so")


def build(verbose: bool = False) -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
