"""Builds the CPU oracle library (plain C, gcc).

Test infrastructure: the oracle is only for the test suite, the smoke check and
the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssu_oracle.c")
LIB = os.path.join(HERE, "libssu_oracle.so")

# -ffp-contract=off: no fused multiply-add, every product and sum is rounded
# on its own, as the oracle's comments state.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-std=c11"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
