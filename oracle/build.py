"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no FMA contraction, no fast-math: the oracle's binary32 steps must be the plain
IEEE operations written in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rmsq_oracle.c")
LIB = os.path.join(HERE, "liboracle_rmsq.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
        "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Build only when the library is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
        os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "rmsq_oracle.h"))
    ):
        build_oracle()
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
