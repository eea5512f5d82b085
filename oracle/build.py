"""Builds liboracle.so, the fp64 CPU oracle, with the host C compiler.

Test infrastructure only: the oracle is built so that the test suite, the
smoke check and the benchmark's CPU-baseline leg can call it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "router_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compiles ``src`` into the shared library ``out``; returns ``out``.
    -O3 for the generic x86-64 target: the library is built on one machine
    and may run on another host CPU, so no -march=native."""
    cmd = ["gcc", "-O3", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
