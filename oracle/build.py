"""Build the C oracle (test infrastructure only).

Compiles ``gdn_oracle.c`` with gcc into ``libgdn_oracle.so`` next to it.  The
flags keep IEEE semantics (no -ffast-math, no FMA contraction) so that every
multiply and add is rounded exactly as written in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-std=c99", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
