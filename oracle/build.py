"""Build the oracle's shared library (test infrastructure only).

The oracle is plain C compiled by gcc with floating-point contraction off,
so every product and sum is rounded exactly as written in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "pic_oracle.c"), os.path.join(HERE, "cdc_oracle.c")]
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle's C sources into liboracle.so next to them; return its path."""
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
