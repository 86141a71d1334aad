"""Builds the oracle's shared library with the host C compiler (gcc, -O2, OpenMP)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "msa_oracle.c")


def library_path() -> str:
    return os.path.join(HERE, "libmsa_oracle.so")


def build(verbose: bool = False, src: str = SOURCE, out: str | None = None) -> str:
    out = out or library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
