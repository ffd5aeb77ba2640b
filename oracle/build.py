"""Builds the C++ oracle (test infrastructure) with g++ into oracle/.

``python -m oracle.build`` writes ``oracle/libmcsoracle.so``. ``build(mutant=k,
out=path)`` writes a copy with planted mistake k (see ORC_MUTANT in
mcsparse_oracle.cpp), which the CPU tests use to show that the pins catch it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mcsparse_oracle.cpp")
LIB = os.path.join(HERE, "libmcsoracle.so")
CXX = os.environ.get("CXX_ORACLE", "g++")

# plain IEEE float64: no fast-math, no contraction into fused multiply-adds
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-Wall", "-Wextra"]


def build(mutant: int = 0, out: str | None = None, verbose: bool = True) -> str:
    out = out or LIB
    tmp = out + ".tmp"
    cmd = [CXX, *FLAGS, f"-DORC_MUTANT={int(mutant)}", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose and mutant == 0:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
