"""Builds liboracle.so from ssd_oracle.c with gcc (host only, OpenMP).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(out=LIB, src=SRC, defines=(), werror=True):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           *(["-Werror"] if werror else []),
           *[f"-D{d}" for d in defines], src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_oracle())
