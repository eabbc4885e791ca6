"""Compile the C oracle (plain gcc, no fast-math) into oracle/liboracle.so.

Test infrastructure only.  ``build(mutant=n)`` writes a separate library with
one deliberate mistake planted, which the test suite uses to show that the
oracle's pins catch it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")


def lib_path(mutant: int = 0) -> str:
    if mutant:
        return os.path.join(HERE, "_mutants", f"liboracle_m{mutant}.so")
    return os.path.join(HERE, "liboracle.so")


def build(mutant: int = 0, quiet: bool = True) -> str:
    out = lib_path(mutant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
           f"-DORACLE_MUTANT={mutant}", SRC, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0, quiet=False))
