"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False, extra=(), src=None, out=None):
    """Compile vrt_oracle.c; no fast-math and no contraction, as the recipe requires."""
    src = src or os.path.join(HERE, "vrt_oracle.c")
    out = out or LIB
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-I", HERE, src, "-o", out + ".tmp", "-lm", *extra]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
