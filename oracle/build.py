"""Build the CPU oracle's shared library (plain C, gcc).

TEST INFRASTRUCTURE ONLY: the oracle is loaded by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

# -ffp-contract=off: no fused multiply-add may change a rounding the definitions fix;
# no -ffast-math: IEEE semantics, NaN / inf / signed zero and nearbyint() ties-to-even hold.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
