"""Build the CPU oracle library (plain C, fp64, OpenMP).

Test infrastructure only: the test-suite, the smoke check and the CPU-baseline leg of the
benchmark are the only users of the oracle.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvrope_oracle.c")
LIB = os.path.join(HERE, "libkvrope_oracle.so")

# -ffp-contract=off: no fused multiply-add, so every product and sum is rounded on its
# own, exactly as written in the C source.  -O3 without -ffast-math vectorises only loops
# whose sums stay in source order (independent accumulators side by side).
CFLAGS = ["-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
