"""Compile the fp64 CPU oracle (test infrastructure) into oracle/libgdn_oracle.so.

Plain gcc; no GPU code is involved.  Run as ``python oracle/build.py`` or via
``build()`` in the package entry file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
# GDN_ORACLE_PATH points the tests at another build of the same source
LIB = os.environ.get("GDN_ORACLE_PATH", os.path.join(HERE, "libgdn_oracle.so"))


def build(verbose: bool = False, mutant: int = 0, out: str = None) -> str:
    """Compile the oracle to ``out`` (default LIB).  ``mutant`` > 0 plants that
    numbered mistake (ORACLE_MUTANT in gdn_oracle.c) for the mutation test only."""
    out = out or LIB
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
           "-Wall", "-Wextra", "-DORACLE_MUTANT=%d" % mutant, "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
